"""Byte offsets of the regions of a pa_attention workspace, restated on the
host for tests that read a workspace back after a call.

libpa sizes its workspace from the host-visible bounds alone (number of
sequences, heads, the longest context and query run).  This module restates
that rule so a test can find, for example, the decode's per-(sequence, KV
head) ticket counters and check that a call left them at zero.  A test that
uses it also compares ``total`` with ``pa_attention_workspace_size``, so a
change of the library's layout that this copy misses fails loudly.
"""
from __future__ import annotations

import math

BLOCK = 16
DECODE_ROWS = 8          # most query rows per (sequence, KV head) the decode takes
MIN_CHUNK = 4            # least (KV head, block) units per decode wave
CASCADE_MIN_BLOCKS = 4   # shared full blocks a shared-prefix group needs
PREFIX_CHUNKS = 8        # workgroups per (group, KV head) at most
CHUNK_TILES = 16         # 64-key tiles per prefix chunk, at least
REC_FLOATS = 132         # (acc[128], m, l, 2 pad) per partial record


def _a256(x: int) -> int:
    return (x + 255) // 256 * 256


def min_slice(T: int) -> int:
    """Least decode slice, in blocks, for a longest pair of T blocks: ceil(sqrt(T)/2)."""
    return (math.isqrt(T) + 1) // 2


def plan_decode(num_seqs, num_q_heads, num_kv_heads, max_context_len, max_query_len):
    """(rows, waves) of the decode kernel a call launches (rows 0: none)."""
    G = num_q_heads // num_kv_heads
    if G > DECODE_ROWS or num_seqs <= 0 or max_query_len <= 0:
        return 0, 0
    need = min(G * max_query_len, DECODE_ROWS)
    rows = 1
    while rows < need:
        rows *= 2
    per_simd = 2 if rows <= 2 else 1
    max_blocks = -(-max_context_len // BLOCK)
    bound = num_seqs * num_kv_heads * max_blocks
    chunk = max(min_slice(min(max_blocks, 2**31 - 1)), MIN_CHUNK)
    waves = max(1, min(-(-bound // chunk), per_simd * 1024))
    return rows, waves


def workspace_layout(num_seqs, num_q_heads, num_kv_heads, max_context_len, max_query_len,
                     min_zero_bytes=0):
    """Offsets (bytes) of every region, their sizes where a test needs them,
    and the total.  The zero region (the shared-prefix plan's item count at 0,
    the decode's ticket counters at 256) comes first; ``min_zero_bytes``
    reserves a larger one, as the library's static scratch array does."""
    G = num_q_heads // num_kv_heads
    rows, waves = plan_decode(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                              max_query_len)
    prefill = max_query_len * G > DECODE_ROWS and num_seqs > 0
    cascade = (rows > 0 and not prefill and num_seqs >= 2
               and max_context_len > CASCADE_MIN_BLOCKS * BLOCK)
    max_items = 0
    if cascade:
        cap = (max_context_len - 1) // BLOCK
        tiles = (cap * BLOCK + 63) // 64
        chunks = min(PREFIX_CHUNKS, max(1, tiles // CHUNK_TILES))
        max_items = (num_seqs // 2) * chunks * num_kv_heads
    split = rows > 0 and waves > 1
    lay = {"rows": rows, "waves": waves, "cascade": cascade, "prefill": prefill,
           "max_items": max_items, "item_count": 0, "counters": 256,
           "counters_bytes": num_seqs * num_kv_heads * 4 if split else 0}
    zero = 0
    if cascade or split or prefill:
        zero = 256 + _a256(num_seqs * num_kv_heads * 4)
    if zero < min_zero_bytes:
        zero = _a256(min_zero_bytes)
    lay["zero_bytes"] = zero
    off = zero
    lay["starts"] = off
    off += _a256(num_seqs * 2 * 4) if cascade else 0
    lay["items"] = off
    off += _a256(max_items * 8 * 4) if cascade else 0
    lay["prefix"] = off
    off += _a256(num_seqs * num_q_heads * PREFIX_CHUNKS * REC_FLOATS * 4) if cascade else 0
    lay["records"] = off
    off += waves * 2 * rows * REC_FLOATS * 4 if split else 0
    lay["queue"] = off
    off += 256 if prefill else 0
    lay["order"] = off
    off += _a256(num_seqs * 4) if prefill else 0
    lay["total"] = off
    return lay
