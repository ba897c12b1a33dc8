def expert_params(d_model: int, d_ff: int) -> int:
    """Parameters of one SwiGLU expert (gate, up, down; no biases): 3 * d * d_ff."""
    return 3 * d_model * d_ff
