"""CPU oracle of the pixel content key used by the vision-embedding cache.

TEST INFRASTRUCTURE ONLY (like ``vit_oracle``): only ``tests/`` may import it.
It shares no code with the HIP library.

The pages name a vision-embedding cache shared across requests ("vLLM
multimodal inference | ViT performance optimisation", section 2.3) but no key;
the key taken here is a 128-bit content key of an item's uint8
pixels.  With the item's L pixel bytes read as L/8 little-endian 64-bit words
w_k (L is a multiple of 16 for every valid item), lane j is

    key_j = mix(S_j ^ (L * G_j)),   S_j = sum_k mix(w_k + (k + 1) * G_j)  (mod 2^64)

with G_0 = 0x9e3779b97f4a7c15, G_1 = 0xd1b54a32d192ed03 and mix the 64-bit
finaliser of SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014).  The cache also compares the grid.
"""

import numpy as np

G = (np.uint64(0x9E3779B97F4A7C15), np.uint64(0xD1B54A32D192ED03))
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def mix64(z):
    """SplitMix64's finaliser on uint64 (array or scalar), arithmetic mod 2^64."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64_stream(seed: int, n: int) -> np.ndarray:
    """The first n outputs of the SplitMix64 generator from `seed` (state += G_0, output mix(state))."""
    with np.errstate(over="ignore"):
        states = np.uint64(seed) + G[0] * np.arange(1, n + 1, dtype=np.uint64)
    return mix64(states)


def item_key(pixels: np.ndarray) -> tuple:
    """(key_0, key_1) of one item's uint8 pixel bytes (any shape, C order)."""
    b = np.ascontiguousarray(pixels, dtype=np.uint8).reshape(-1)
    assert b.size % 16 == 0, "item pixel bytes are a multiple of 16"
    w = b.view("<u8").astype(np.uint64)
    k1 = np.arange(1, w.size + 1, dtype=np.uint64)
    out = []
    with np.errstate(over="ignore"):
        for g in G:
            s = np.sum(mix64(w + k1 * g), dtype=np.uint64)
            out.append(int(mix64(s ^ (np.uint64(b.size) * g))))
    return tuple(out)
