"""Rotation-FLOP accounting of one prefill query tile (test infrastructure only).

LazyAttention summary, "Technical Implementation" (prefilling phase): instead of
rotating cached keys twice (back to zero, then to the target position) the
kernel applies a single relative rotation per query tile, which costs about
3/(4M) of the tile's attention FLOPs, ~0.59% at M = 128.

Counted from the definitions used elsewhere in this oracle:
  * one RoPE rotation of a key row of D dims rotates D/2 pairs, each pair
    costing 4 multiplies + 2 adds (rotate.py);
  * one query tile of M rows against N keys costs 2 M N D FLOPs for Q K^T and
    2 M N D FLOPs for P V.
"""

FLOPS_PER_PAIR = 4 + 2


def rotation_flops(N: int, D: int, rotations_per_key: int = 1) -> int:
    return rotations_per_key * N * (D // 2) * FLOPS_PER_PAIR


def attention_flops(M: int, N: int, D: int) -> int:
    return 2 * M * N * D + 2 * M * N * D


def rotation_overhead(M: int, N: int = 64, D: int = 128, rotations_per_key: int = 1) -> float:
    """Rotation FLOPs / attention FLOPs for one (M-row query tile, N-key tile)."""
    return rotation_flops(N, D, rotations_per_key) / attention_flops(M, N, D)
