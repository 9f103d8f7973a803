"""Packed (block id, logical offset) metadata word -- independent encoder/decoder.

The LazyAttention summary ("Technical Implementation", decoding phase) says the
block ID and offset are bit-packed into a single register so the kernel needs
no extra global loads, but gives no bit layout. The layout taken here:

  bits [16:0]  physical block id, 0 .. 2^17 - 1
  bits [31:17] delta = offset - t*B as 15-bit two's complement, -2^14 .. 2^14-1

where t is the entry's index inside its sequence's block table and offset is
the logical position of the block's slot 0. A block id needs 17 bits for pools
of ~128k blocks and absolute positions need 16, so an absolute offset does not
fit beside the id; delta does, and it stays constant over blocks that sit
back-to-back, so "the offset changes" coincides with a document boundary.

Written with plain integer arithmetic (no shared code with the product's
encoder), test infrastructure only.
"""
import numpy as np

ID_BITS = 17
DELTA_BITS = 15
ID_MAX = (1 << ID_BITS) - 1          # 131071
DELTA_MIN = -(1 << (DELTA_BITS - 1))  # -16384
DELTA_MAX = (1 << (DELTA_BITS - 1)) - 1  # 16383


def _entry_index(block_table: np.ndarray) -> np.ndarray:
    """t for every flat entry: its position inside its own sequence."""
    bt = np.asarray(block_table, dtype=np.int64)
    n = int(bt[-1])
    t = np.arange(n, dtype=np.int64)
    seq = np.searchsorted(bt, t, side="right") - 1
    return t - bt[seq]


def encode_meta(block_ids, offsets, block_table, B: int) -> np.ndarray:
    """Pack per-entry (block id, offset) into uint32 words; ValueError if out of range."""
    ids = np.asarray(block_ids, dtype=np.int64)
    off = np.asarray(offsets, dtype=np.int64)
    t = _entry_index(block_table)
    if ids.shape != off.shape or ids.shape != t.shape:
        raise ValueError("block_ids/offsets must have block_table[-1] entries")
    delta = off - t * B
    if np.any(ids < 0) or np.any(ids > ID_MAX):
        raise ValueError("block id out of range")
    if np.any(delta < DELTA_MIN) or np.any(delta > DELTA_MAX):
        raise ValueError("offset delta out of range")
    d15 = delta % (1 << DELTA_BITS)           # two's complement in 15 bits
    words = ids + d15 * (1 << ID_BITS)
    return words.astype(np.uint32)


def decode_meta(words, block_table, B: int):
    """Inverse of encode_meta: (block ids int64, offsets int64)."""
    w = np.asarray(words, dtype=np.uint32).astype(np.int64)
    ids = w % (1 << ID_BITS)
    d15 = w // (1 << ID_BITS)
    delta = np.where(d15 >= (1 << (DELTA_BITS - 1)), d15 - (1 << DELTA_BITS), d15)
    t = _entry_index(block_table)
    return ids, delta + t * B
