"""Storage accounting of the compressed cache (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Ingredients (QuantWM v2 App. D.1; rainbus digest method step (3), Sec. 5.1):
INT2 residual codes, a uint8 centroid index, per-group scale and bit-packed
INT2 zero-points, PSAC coefficients C in INT8 with U_r in BF16, BF16
centroid tables.  The pages' memory figure (Fig. 6 / Sec. 5.5):
LongCat-Video 21.709 GiB -> 3.625 GiB for 93 frames.
"""
from __future__ import annotations


def key_bits(d: int = 128, group: int = 64, r: int = 8, psac: bool = True) -> int:
    G = d // group
    bits = d * 2 + 8 + G * 16 + G * 2        # codes, index, fp16 scales, zero-points
    if psac:
        bits += r * 8 + 16                   # INT8 coefficients + fp16 scale
    return bits


def value_bits(d: int = 128, group: int = 64) -> int:
    G = d // group
    return d * 2 + 8 + G * 16 + G * 2


def bits_per_token_head(d: int = 128, group: int = 64, r: int = 8) -> int:
    return key_bits(d, group, r) + value_bits(d, group)


def bf16_bits_per_token_head(d: int = 128) -> int:
    return 2 * d * 16


def ratio_per_token(d: int = 128, group: int = 64, r: int = 8) -> float:
    return bf16_bits_per_token_head(d) / bits_per_token_head(d, group, r)


def table_bytes(d: int = 128, n_c: int = 256, r: int = 8) -> int:
    """Per (chunk, head): K and V centroid tables (bf16) + U_r (bf16)."""
    return 2 * n_c * d * 2 + d * r * 2


def resident_ratio(tokens_per_chunk: int, n_chunks: int, d: int = 128, n_c: int = 256,
                   r: int = 8) -> float:
    """BF16 bytes / compressed bytes including the per-(chunk, head) tables."""
    T = tokens_per_chunk * n_chunks
    comp = T * bits_per_token_head(d, 64, r) / 8 + n_chunks * table_bytes(d, n_c, r)
    return T * bf16_bits_per_token_head(d) / 8 / comp
