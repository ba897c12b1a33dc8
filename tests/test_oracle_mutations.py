"""Plant plausible mistakes in the oracle and check that a pin catches each one.

Every mutation is applied to the CPU oracle only, with monkeypatch, and
undone after the test.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
import test_oracle_pins as pins

F64 = np.float64


def _fails(fn):
    with pytest.raises(AssertionError):
        fn()


def test_tie_break_to_higher_index_is_caught(monkeypatch):
    def bad(scores, k):
        s = np.asarray(scores, dtype=F64)
        E = s.shape[-1]
        rev = np.argsort(-s[..., ::-1], axis=-1, kind="stable")  # ties -> higher index
        return (E - 1 - rev)[..., :k]
    monkeypatch.setattr(O, "topk_order", bad)
    _fails(pins.test_topk_bruteforce_exhaustive_with_ties)


def test_gate_up_swapped_is_caught(monkeypatch):
    orig = O.swiglu_expert
    monkeypatch.setattr(O, "swiglu_expert", lambda X, g, u, d, round_h: orig(X, u, g, d, round_h))
    _fails(pins.test_e1_k1_is_dense_swiglu_ffn)


def test_transposed_down_is_caught(monkeypatch):
    def bad(X, g, u, d, round_h):
        X = np.atleast_2d(np.asarray(X, dtype=F64))
        h = O.silu(X @ np.asarray(g, F64).T) * (X @ np.asarray(u, F64).T)
        dd = np.asarray(d, F64)
        return h @ (dd if dd.shape[0] == dd.shape[1] else dd.T)  # wrong when square
    monkeypatch.setattr(O, "swiglu_expert", bad)

    def square_case():
        rng = np.random.default_rng(0)
        x = rng.standard_normal((9, 16))
        wg, wu, wd, _ = pins.rand_layer(rng, 1, 16, 16)
        y = O.moe_layer(x, rng.standard_normal((1, 16)), wg, wu, wd, 1).y
        np.testing.assert_allclose(y, pins.torch_swiglu(x, wg[0], wu[0], wd[0]), rtol=1e-12)
    _fails(square_case)


def test_fraction_over_tokens_is_caught(monkeypatch):
    def bad(counts, prob_sum, n_tokens, top_k):
        c, p = np.asarray(counts, F64), np.asarray(prob_sum, F64)
        return float(c.shape[0] * np.sum(c / n_tokens * p / n_tokens))
    monkeypatch.setattr(O, "balance_stat", bad)
    _fails(pins.test_balance_stat_uniform_probs_is_one)


def test_dropped_shared_term_is_caught(monkeypatch):
    orig = O.forward_per_token
    monkeypatch.setattr(O, "forward_per_token",
                        lambda *a, shared=None, **kw: orig(*a, shared=None, **kw))
    _fails(pins.test_shared_expert_adds_dense_ffn)


def test_missing_renormalisation_is_caught(monkeypatch):
    orig = O.route
    monkeypatch.setattr(O, "route", lambda x, W, k, logit_bias=None, select_bias=None, renormalize=True:
                        orig(x, W, k, logit_bias, select_bias, False))
    _fails(pins.test_renormalised_weights_sum_to_one_and_special_k)


def test_capacity_keeping_last_copies_is_caught(monkeypatch):
    def bad(idx, E, C):
        flat = np.asarray(idx).reshape(-1)
        keep = np.ones(flat.shape[0], dtype=bool)
        if C <= 0:
            return keep
        for e in range(E):
            where = np.nonzero(flat == e)[0]
            keep[where[: max(0, len(where) - C)]] = False  # keeps the last C
        return keep
    monkeypatch.setattr(O, "capacity_keep", bad)
    _fails(lambda: pins.test_capacity_bruteforce(2))


def test_softmax_without_exp_is_caught(monkeypatch):
    def bad(l):
        l = np.asarray(l, F64) - np.min(l, axis=-1, keepdims=True)
        return l / l.sum(axis=-1, keepdims=True)
    monkeypatch.setattr(O, "softmax", bad)
    _fails(pins.test_softmax_matches_scipy_and_sums_to_one)


def test_weights_from_biased_scores_is_caught(monkeypatch):
    def bad(x, W, k, logit_bias=None, select_bias=None, renormalize=True):
        p = O.softmax(O.router_logits(x, W, logit_bias))
        s = p if select_bias is None else p + np.asarray(select_bias)[None, :]
        idx = O.topk_order(s, k)
        w = np.take_along_axis(s, idx, axis=1)  # weights from the biased score: wrong
        return O.Routing(idx=idx, w=w, probs=p, gap=np.zeros(p.shape[0]))
    monkeypatch.setattr(O, "route", bad)
    _fails(pins.test_selection_bias_picks_but_does_not_weight)


def test_bf16_truncation_is_caught(monkeypatch):
    def bad(a):
        a = np.asarray(a, F64)
        m, e = np.frexp(a)
        return np.ldexp(np.trunc(m * 256) / 256, e)
    monkeypatch.setattr(O, "bf16_round", bad)
    _fails(pins.test_bf16_round_matches_torch_on_fp32)


def test_fp8_ties_away_from_zero_is_caught(monkeypatch):
    orig = O.fp8_e4m3_encode

    def bad(v):
        a = np.asarray(v, dtype=F64)
        # nudge every magnitude up by a hair: ties now round away from zero
        return orig(np.sign(a) * np.nextafter(np.abs(a), np.inf))
    monkeypatch.setattr(O, "fp8_e4m3_encode", bad)
    _fails(pins.test_fp8_encode_is_nearest_even_bruteforce)


def test_fp8_scale_per_column_is_caught(monkeypatch):
    orig = O.quantize_fp8_rows
    monkeypatch.setattr(O, "quantize_fp8_rows", lambda w: tuple(a.T if a.ndim == 2 else a for a in orig(np.asarray(w).T)))
    _fails(pins.test_fp8_row_quantisation_invariants)


def test_z_loss_without_square_is_caught(monkeypatch):
    def bad(logits):
        l = np.asarray(logits, dtype=F64)
        if l.shape[0] == 0:
            return 0.0
        m = l.max(axis=1, keepdims=True)
        return float(np.mean(m[:, 0] + np.log(np.exp(l - m).sum(axis=1))))
    monkeypatch.setattr(O, "z_loss", bad)
    _fails(pins.test_z_loss_closed_forms_and_scipy)


def test_bias_update_wrong_direction_is_caught(monkeypatch):
    orig = O.update_select_bias
    monkeypatch.setattr(O, "update_select_bias", lambda b, c, n, k, g: orig(b, c, n, k, -g))
    _fails(pins.test_select_bias_update_bruteforce)


def test_int4_ties_away_from_zero_is_caught(monkeypatch):
    orig = O.quantize_int4_rows

    def bad(w):
        q, s = orig(w)
        w32 = np.asarray(w, dtype=np.float32)
        r = (w32 / np.where(s > 0, s, np.float32(1))[:, None]).astype(np.float64)
        half = np.abs(r - np.trunc(r)) == 0.5
        q = np.where(half & (s[:, None] > 0), np.clip(np.trunc(r) + np.sign(r), -7, 7), q).astype(np.int8)
        return q, s
    monkeypatch.setattr(O, "quantize_int4_rows", bad)
    _fails(pins.test_int4_quantisation_is_nearest_even_bruteforce)


def test_int4_scale_over_eight_is_caught(monkeypatch):
    # reading the int4 range as [-8, 7] with scale = max / 8
    def bad(w):
        w32 = np.asarray(w, dtype=np.float32)
        s = (np.max(np.abs(w32), axis=1) / np.float32(8)).astype(np.float32)
        r = w32 / np.where(s > 0, s, np.float32(1))[:, None]
        return np.clip(np.rint(r), -8, 7).astype(np.int8), s
    monkeypatch.setattr(O, "quantize_int4_rows", bad)
    _fails(pins.test_int4_row_quantisation_invariants)


def test_int4_natural_nibble_order_is_caught(monkeypatch):
    monkeypatch.setattr(O, "_INT4_SHIFT", 4 * np.arange(8))
    _fails(pins.test_int4_packing_matches_worked_block_and_round_trips)


def test_int4_offset_binary_field_is_caught(monkeypatch):
    # codes stored as q + 8 instead of sign and magnitude
    monkeypatch.setattr(O, "_int4_field", lambda q: np.asarray(q, dtype=np.int64) + 8)
    _fails(pins.test_int4_packing_matches_worked_block_and_round_trips)


# ---------------------------------------------------------------- backward oracle
import test_oracle_backward as bpins
from oracle import moe_backward as OB


def test_backward_silu_grad_without_second_term_is_caught(monkeypatch):
    monkeypatch.setattr(OB, "silu_grad", lambda z: OB.sigmoid(z))
    _fails(lambda: bpins.test_backward_matches_finite_differences(True))


def test_backward_renormalisation_without_projection_is_caught(monkeypatch):
    monkeypatch.setattr(OB, "renorm_backward", lambda dw, w, ssum: dw / ssum)
    _fails(lambda: bpins.test_backward_matches_finite_differences(True))


def test_backward_softmax_without_centering_is_caught(monkeypatch):
    monkeypatch.setattr(OB, "softmax_backward", lambda p, dp: p * dp)
    _fails(lambda: bpins.test_backward_matches_finite_differences(False))


def test_backward_dropped_copies_sending_gradient_is_caught(monkeypatch):
    orig_group = OB._grouping
    monkeypatch.setattr(OB, "_grouping", lambda idx, E, capacity=0: orig_group(idx, E, 0))
    _fails(lambda: bpins.test_backward_matches_finite_differences(True))


def test_gap_on_unbiased_probs_is_caught(monkeypatch):
    orig = O.route

    def bad(x, W, k, logit_bias=None, select_bias=None, renormalize=True):
        r = orig(x, W, k, logit_bias, select_bias, renormalize)
        if k < r.probs.shape[1]:
            srt = -np.sort(-r.probs, axis=1)
            r.gap = srt[:, k - 1] - srt[:, k]
        return r
    monkeypatch.setattr(O, "route", bad)
    _fails(pins.test_route_gap_planted_scores)


def test_gap_one_slot_off_is_caught(monkeypatch):
    orig = O.route

    def bad(x, W, k, logit_bias=None, select_bias=None, renormalize=True):
        r = orig(x, W, k, logit_bias, select_bias, renormalize)
        s = r.probs + (0.0 if select_bias is None else np.asarray(select_bias)[None, :])
        srt = -np.sort(-s, axis=1)
        if 2 <= k < s.shape[1]:
            r.gap = srt[:, k - 2] - srt[:, k - 1]
        return r
    monkeypatch.setattr(O, "route", bad)
    _fails(pins.test_route_gap_planted_scores)


def test_forced_weights_from_biased_scores_is_caught(monkeypatch):
    def bad(r, idx, renormalize=True):
        idx = np.asarray(idx, dtype=np.int64)
        w = np.take_along_axis(r.probs + 0.01, idx, axis=1)   # a shifted score instead of p
        if renormalize:
            w = w / w.sum(axis=1, keepdims=True)
        return O.Routing(idx=idx, w=w, probs=r.probs, gap=r.gap)
    monkeypatch.setattr(O, "forced_routing", bad)
    _fails(pins.test_forced_routing_weights_bruteforce)


def test_band_without_error_bound_is_caught(monkeypatch):
    orig = O.fp32_dot_bound
    monkeypatch.setattr(O, "fp32_dot_bound", lambda X, W, chunk=16, parts=8, lam=O.LAMBDA:
                        0.0 * orig(X, W, chunk, parts, lam))
    monkeypatch.setattr(O, "U32", 0.0)
    _fails(pins.test_h_band_contains_fp32_evaluations)


def test_band_one_sided_range_is_caught(monkeypatch):
    # only roundings at or above the oracle's own counted as correct
    orig = O.h_rounding_band

    def bad(*a, **kw):
        b = orig(*a, **kw)
        b.lo = b.ref.copy()
        b.amb = b.lo < b.hi
        return b
    monkeypatch.setattr(O, "h_rounding_band", bad)
    _fails(pins.test_h_band_planted_midpoint)


def test_weights_paired_with_wrong_slot_are_caught(monkeypatch):
    orig = O.forward_per_token
    monkeypatch.setattr(O, "forward_per_token",
                        lambda x, idx, w, keep, *a, **kw: orig(x, idx, np.roll(w, 1, axis=1), keep, *a, **kw))
    _fails(lambda: pins.test_y_superposition_over_experts(0, True, False))


def test_dropped_copies_contributing_are_caught(monkeypatch):
    orig = O.forward_per_token
    monkeypatch.setattr(O, "forward_per_token",
                        lambda x, idx, w, keep, *a, **kw: orig(x, idx, w, np.ones_like(keep), *a, **kw))
    _fails(lambda: pins.test_y_superposition_over_experts(9, False, False))


def test_expert_weights_off_by_one_are_caught(monkeypatch):
    class Shift:
        def __init__(self, a):
            self.a = a

        def __getitem__(self, e):
            return self.a[(e + 1) % len(self.a)]

        def __len__(self):
            return len(self.a)

    orig = O.forward_per_token
    monkeypatch.setattr(O, "forward_per_token",
                        lambda x, idx, w, keep, g, u, d, *a, **kw: orig(x, idx, w, keep, Shift(g), Shift(u), Shift(d),
                                                                         *a, **kw))
    _fails(lambda: pins.test_y_superposition_over_experts(0, True, False))
    _fails(lambda: pins.test_y_invariant_under_expert_relabelling(0))


def test_logit_bias_left_with_its_index_is_caught(monkeypatch):
    # the logit bias applied by position after the experts were relabelled would break the invariance
    orig = O.route
    monkeypatch.setattr(O, "route", lambda x, W, k, logit_bias=None, select_bias=None, renormalize=True:
                        orig(x, W, k, None if logit_bias is None else np.sort(logit_bias), select_bias, renormalize))
    _fails(lambda: pins.test_y_invariant_under_expert_relabelling(0))
