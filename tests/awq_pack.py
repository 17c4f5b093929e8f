"""Test-side AWQ packer written from the golden words (tests/golden/awq_words.txt).

Inverse direction of the oracle's unpacking; checked against the golden words
before any use.  Not part of the oracle or of the HIP path.
"""
import numpy as np

# nibble i of a word holds logical column NIBBLE_COLUMN[i] of its group of eight
NIBBLE_COLUMN = (0, 2, 4, 6, 1, 3, 5, 7)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """codes [..., N] in 0..15 -> int32 words [..., N/8]."""
    codes = np.asarray(codes, np.uint32)
    *lead, N = codes.shape
    groups = codes.reshape(*lead, N // 8, 8)
    word = np.zeros((*lead, N // 8), np.uint32)
    for i, col in enumerate(NIBBLE_COLUMN):
        word |= (groups[..., col] & 0xF) << np.uint32(4 * i)
    return word.view(np.int32)
