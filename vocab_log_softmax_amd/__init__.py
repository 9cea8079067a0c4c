"""Fused row-wise log-softmax heads (logprobs, entropy, KL, softcap) for MI355X."""
