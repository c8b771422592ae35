"""Row bookkeeping for the tests (independent of the library and the oracle).

With M query tokens per sequence, the tokens are the sequence's last M
positions and token m attends to the keys at positions t <= L - M + m (the
causal rule the multi-token calls document): this is how many keys that is.
"""


def causal_len(L: int, M: int, m: int) -> int:
    """Keys query token m (of M) sees in a length-L sequence, clamped to [0, L]."""
    return max(0, min(L, L - M + m + 1))


def used_partitions(L: int, M: int, m: int, PS: int) -> int:
    """Partitions of PS tokens that hold at least one of those keys."""
    return -(-causal_len(L, M, m) // PS)
