"""The entries the global top-M engine samples to place its first window, by its documented rule, so that tests can
plant misleading values there and drive the engine's fallback classification."""
import numpy as np


def sampled_entries(n):
    """Entries the top-M engine samples to place its first window (its documented rule: S = min(65536, n // 4)
    strata, the float4 at fraction ((40503 j + 17) mod 2^16) / 2^16 of stratum j)."""
    n4 = n // 4
    S = min(65536, n4)
    j = np.arange(S, dtype=np.int64)
    pos4 = ((j * 65536 + ((j * 40503 + 17) & 0xFFFF)) * n4) // (S * 65536)
    return (4 * pos4[:, None] + np.arange(4)[None, :]).reshape(-1)
