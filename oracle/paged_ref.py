"""Plain fp64 CPU oracle for generalized paged attention.

TEST INFRASTRUCTURE ONLY.  This module exists to check the HIP path; it is
imported by ``tests/``, by ``__graft_entry__.smoke()`` and by the bench's
``cpu_baseline`` leg, and by nothing else.  The product path never calls it
and shares no code with it.

What it computes, and where the pages define it:

* ``kv_write_ref`` -- each new token's K and V row is copied into the slot
  its sequence appends to (PagedAttention explainer, "ブロックテーブルによる
  メモリ管理": a new token goes into the current physical block while it has
  room, otherwise into a freshly allocated one).  A slot is
  ``physical_block * 16 + offset``; ``-1`` skips the token.  Done on the raw
  16-bit patterns, so it is exact.
* ``attention_ref`` -- ``softmax(Q K^T * scale) V`` (PagedAttention
  explainer, "PagedAttentionアルゴリズム", the attention equation; KV-cache
  textbook ch.1), with K and V reached through the block table one 16-token
  block at a time, and a causal mask on the new tokens: the ``n`` new query
  rows of a sequence with ``C`` visible keys are its last ``n`` positions,
  so row ``i`` sees keys ``0 .. C-n+i`` (Pensieve explainer, "汎化
  PagedAttentionカーネル": several new tokens over a partly cached,
  non-contiguous history, with a fused causal mask).
* ``attention_blockwise_ref`` -- the per-block form of the same result:
  ``A_j = exp(q K_j^T/sqrt(d)) / sum_i sum_k exp(q k_{i,k}^T/sqrt(d))`` and
  ``o = sum_j A_j V_j`` (PagedAttention explainer, "PagedAttentionアルゴリズム",
  the blockwise equation).
* ``attention_split_merge_ref`` -- the key range is cut into partitions,
  each kept as (running max m, sum l, unnormalised output acc), and merged
  by rescaling with ``exp(m_p - M)``; the logsumexp ``L = m + log(l)``
  carries the same statistics (KV-cache textbook ch.6, FlashAttention-2).
  The vLLM kernel's per-block scores followed by an aggregation step
  (PagedAttention explainer, "実装のポイント") is this merge.
* closed forms for KV size and block accounting (Pensieve explainer,
  "KVキャッシュのメモリ管理"; KV-cache textbook ch.3; PagedAttention
  explainer, "PagedAttentionアルゴリズム" and "ブロックテーブルによるメモリ管理").

Conventions the pages leave open, taken here (shared with the HIP path as a
convention, not as code): pools are ``[num_blocks, num_kv_heads, 16, d]``;
query head ``h`` reads KV head ``h // (Hq // Hkv)``; ``context_lens`` counts
the new tokens too; block-table entries past a sequence's last block are
never read.

Every function here is pinned by ``tests/test_oracle_*.py`` against things
other than itself: hand-derived values, brute-force attention over a
contiguous copy, torch's CPU ``scaled_dot_product_attention`` in float64,
special cases with closed-form answers, permutation and sharing invariance,
and the numbers the pages print.
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


# ----------------------------------------------------------------------------
# bit patterns -> float64
# ----------------------------------------------------------------------------
def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of an array of fp16 or bf16 bit patterns."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def kv_bytes_per_token(num_layers: int, hidden: int, bytes_per_elem: int) -> int:
    """KV-cache bytes one token costs: layers x hidden x 2 (K and V) x bytes.

    Pensieve explainer, "KVキャッシュのメモリ管理", the M_kv equation.
    """
    return num_layers * hidden * 2 * bytes_per_elem


def kv_cache_elements(batch: int, num_layers: int, seq_len: int, head_dim: int,
                      num_heads: int) -> int:
    """Elements of a KV cache: 2 x batch x layers x seq_len x head_dim x heads.

    KV-cache textbook ch.3, the element-count formula.
    """
    return 2 * batch * num_layers * seq_len * head_dim * num_heads


def num_blocks(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """N = ceil(n / B), the blocks a sequence of n tokens occupies.

    PagedAttention explainer, "PagedAttentionアルゴリズム".
    """
    return -(-int(num_tokens) // int(block_size))


def internal_fragmentation(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Unused slots in a sequence's last block (at most B - 1).

    PagedAttention explainer, "ブロックテーブルによるメモリ管理".
    """
    return num_blocks(num_tokens, block_size) * block_size - int(num_tokens)


# ----------------------------------------------------------------------------
# kv_write
# ----------------------------------------------------------------------------
def kv_write_ref(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
                 v_new: np.ndarray, slot_mapping: np.ndarray,
                 block_size: int = BLOCK_SIZE):
    """Copy of (k_pool, v_pool) with every new token's rows placed in its slot.

    Pools ``[NB, Hkv, B, D]`` and new rows ``[T, Hkv, D]`` are 16-bit patterns;
    nothing is converted.  Slots must be distinct and inside the pool.
    """
    k_out = np.array(k_pool, dtype=np.uint16, copy=True)
    v_out = np.array(v_pool, dtype=np.uint16, copy=True)
    nb = k_out.shape[0]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    written = slots[slots >= 0]
    if written.size:
        assert np.unique(written).size == written.size, "duplicate slots"
        assert int(written.max()) < nb * block_size, "slot outside the pool"
    for t in range(slots.shape[0]):
        slot = int(slots[t])
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        k_out[block, :, offset, :] = k_new[t]
        v_out[block, :, offset, :] = v_new[t]
    return k_out, v_out


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def gather_keys_values(k_pool: np.ndarray, v_pool: np.ndarray, table_row: np.ndarray,
                       context_len: int, kv_head: int, dtype: str,
                       block_size: int = BLOCK_SIZE):
    """Logical K, V ``[C, D]`` of one sequence and KV head, block by block."""
    C = int(context_len)
    k_rows, v_rows = [], []
    for j in range(num_blocks(C, block_size)):
        phys = int(table_row[j])
        k_rows.append(k_pool[phys, kv_head])
        v_rows.append(v_pool[phys, kv_head])
    if not k_rows:
        D = k_pool.shape[-1]
        return np.zeros((0, D)), np.zeros((0, D))
    K = np.concatenate(k_rows, axis=0)[:C]
    V = np.concatenate(v_rows, axis=0)[:C]
    return bits_to_f64(K, dtype), bits_to_f64(V, dtype)


def _visible_limit(C: int, n: int, rows: np.ndarray) -> np.ndarray:
    """Last key index each new-token row may see (bottom-right causal)."""
    return C - n + np.asarray(rows, dtype=np.int64)


def _softmax_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                    limit: np.ndarray):
    """softmax(scale Q K^T, keys past ``limit`` masked) V, rows of Q independent."""
    X = scale * (Q @ K.T)
    j = np.arange(K.shape[0])
    X[j[None, :] > limit[:, None]] = -np.inf
    m = X.max(axis=1, keepdims=True)
    W = np.exp(X - m)
    l = W.sum(axis=1, keepdims=True)
    W /= l
    return W @ V, W, m[:, 0] + np.log(l[:, 0])


def _group(num_q_heads: int, num_kv_heads: int) -> int:
    assert num_q_heads % num_kv_heads == 0
    return num_q_heads // num_kv_heads


def attention_ref(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                  block_tables: np.ndarray, context_lens: np.ndarray,
                  query_start_loc: np.ndarray, num_kv_heads: int, scale: float,
                  dtype: str, block_size: int = BLOCK_SIZE, return_weights: bool = False,
                  row_chunk: int = 1024):
    """fp64 output ``[Tq, Hq, D]`` (and lse ``[Tq, Hq]``) of paged attention.

    ``q`` holds 16-bit patterns ``[Tq, Hq, D]``.  Sequence ``s`` owns query
    rows ``query_start_loc[s] .. query_start_loc[s+1]-1``; with ``n`` rows and
    ``C = context_lens[s]`` keys, row ``i`` sees keys ``0 .. C-n+i``.
    ``return_weights`` also returns the softmax weights per (s, h) (tiny cases).
    """
    Tq, Hq, D = q.shape
    G = _group(Hq, num_kv_heads)
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    lse = np.zeros((Tq, Hq), dtype=np.float64)
    weights = {}
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    for s in range(len(context_lens)):
        lo, hi = int(qsl[s]), int(qsl[s + 1])
        n, C = hi - lo, int(context_lens[s])
        assert 0 <= n <= C, "need 0 <= n_s <= C_s"
        if n == 0:
            continue
        for g in range(num_kv_heads):
            K, V = gather_keys_values(k_pool, v_pool, block_tables[s], C, g, dtype, block_size)
            for h in range(g * G, (g + 1) * G):
                for r0 in range(0, n, row_chunk):
                    rows = np.arange(r0, min(n, r0 + row_chunk))
                    Q = bits_to_f64(q[lo + rows, h], dtype)
                    o, W, L = _softmax_attend(Q, K, V, scale, _visible_limit(C, n, rows))
                    out[lo + rows, h] = o
                    lse[lo + rows, h] = L
                    if return_weights:
                        weights.setdefault((s, h), []).append(W)
    if return_weights:
        weights = {k: np.concatenate(v, axis=0) for k, v in weights.items()}
        return out, lse, weights
    return out, lse


def attention_ref_sample(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                         block_tables: np.ndarray, context_lens: np.ndarray,
                         query_start_loc: np.ndarray, num_kv_heads: int, scale: float,
                         dtype: str, samples, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """fp64 outputs ``[len(samples), D]`` for chosen ``(token, q_head)`` pairs.

    Same definition as :func:`attention_ref`, evaluated only where asked, so
    full-size workloads can be checked on a sample of their outputs.
    """
    Hq = q.shape[1]
    G = _group(Hq, num_kv_heads)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    res = np.zeros((len(samples), q.shape[2]), dtype=np.float64)
    by_head = {}
    for idx, (t, h) in enumerate(samples):
        s = int(np.searchsorted(qsl, t, side="right") - 1)
        by_head.setdefault((s, int(h) // G), []).append((idx, int(t), int(h)))
    for (s, g), items in by_head.items():
        lo, hi = int(qsl[s]), int(qsl[s + 1])
        n, C = hi - lo, int(context_lens[s])
        K, V = gather_keys_values(k_pool, v_pool, block_tables[s], C, g, dtype, block_size)
        for idx, t, h in items:
            row = np.array([t - lo])
            Q = bits_to_f64(q[t:t + 1, h], dtype)
            o, _, _ = _softmax_attend(Q, K, V, scale, _visible_limit(C, n, row))
            res[idx] = o[0]
    return res


def attention_blockwise_ref(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                            block_tables: np.ndarray, context_lens: np.ndarray,
                            query_start_loc: np.ndarray, num_kv_heads: int, scale: float,
                            dtype: str, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """The per-block equation, one query row at a time.

    For block ``j`` of the sequence the row's unnormalised weights are
    ``exp(scale q K_j^T)``; the denominator sums them over every key of every
    block; ``o = sum_j A_j V_j``.  Masked keys (past the row's causal limit or
    past ``C`` in the last block) contribute nothing.  Numerator and
    denominator are both multiplied by ``exp(-M)`` with ``M`` the row's largest
    logit, which leaves every ``A_j`` unchanged and keeps exp in range.
    """
    Tq, Hq, D = q.shape
    G = _group(Hq, num_kv_heads)
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    for s in range(len(context_lens)):
        lo, hi = int(qsl[s]), int(qsl[s + 1])
        n, C = hi - lo, int(context_lens[s])
        N = num_blocks(C, block_size)
        for h in range(Hq):
            g = h // G
            for i in range(n):
                qv = bits_to_f64(q[lo + i, h], dtype)
                last_key = C - n + i
                logits, values = [], []
                for j in range(N):
                    phys = int(block_tables[s, j])
                    first = j * block_size
                    count = min(block_size, last_key + 1 - first)
                    if count <= 0:
                        break
                    Kj = bits_to_f64(k_pool[phys, g, :count], dtype)
                    Vj = bits_to_f64(v_pool[phys, g, :count], dtype)
                    logits.append(scale * (Kj @ qv))
                    values.append(Vj)
                M = max(float(x.max()) for x in logits)
                denom = sum(float(np.exp(x - M).sum()) for x in logits)
                o = np.zeros(D)
                for x, Vj in zip(logits, values):
                    A_j = np.exp(x - M) / denom
                    o += A_j @ Vj
                out[lo + i, h] = o
    return out


def merge_partitions(parts):
    """Combine per-partition (m, l, acc) into the normalised output.

    ``m`` is a partition's largest logit, ``l = sum exp(x - m)`` and
    ``acc = sum exp(x - m) v``.  With ``M = max_p m_p`` the totals are
    ``l = sum_p l_p exp(m_p - M)`` and ``acc = sum_p acc_p exp(m_p - M)``;
    the output is ``acc / l`` and the logsumexp is ``M + log(l)``.  Empty
    partitions carry ``m = -inf, l = 0`` and drop out.
    """
    live = [(m, l, a) for (m, l, a) in parts if l > 0]
    M = max(m for m, _, _ in live)
    l_tot = sum(l * np.exp(m - M) for m, l, _ in live)
    acc = sum(a * np.exp(m - M) for m, _, a in live)
    return acc / l_tot, M + np.log(l_tot)


def partition_state(x: np.ndarray, V: np.ndarray):
    """(m, l, acc) of one partition from its logits ``x`` and value rows ``V``."""
    if x.size == 0:
        return -np.inf, 0.0, np.zeros(V.shape[-1])
    m = float(x.max())
    p = np.exp(x - m)
    return m, float(p.sum()), p @ V


def attention_split_merge_ref(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                              block_tables: np.ndarray, context_lens: np.ndarray,
                              query_start_loc: np.ndarray, num_kv_heads: int, scale: float,
                              dtype: str, cuts_for, block_size: int = BLOCK_SIZE):
    """Output from partitions of each row's visible keys, merged.

    ``cuts_for(s, h, i, visible)`` returns sorted cut points inside
    ``(0, visible)``; the keys ``[c_k, c_{k+1})`` form partition ``k``.
    Returns (out, lse) like :func:`attention_ref`.
    """
    Tq, Hq, D = q.shape
    G = _group(Hq, num_kv_heads)
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    lse = np.zeros((Tq, Hq), dtype=np.float64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    for s in range(len(context_lens)):
        lo, hi = int(qsl[s]), int(qsl[s + 1])
        n, C = hi - lo, int(context_lens[s])
        for g in range(num_kv_heads):
            K, V = gather_keys_values(k_pool, v_pool, block_tables[s], C, g, dtype, block_size)
            for h in range(g * G, (g + 1) * G):
                for i in range(n):
                    visible = C - n + i + 1
                    qv = bits_to_f64(q[lo + i, h], dtype)
                    x = scale * (K[:visible] @ qv)
                    edges = [0] + [int(c) for c in cuts_for(s, h, i, visible)] + [visible]
                    parts = [partition_state(x[a:b], V[a:b]) for a, b in zip(edges, edges[1:])]
                    o, L = merge_partitions(parts)
                    out[lo + i, h] = o
                    lse[lo + i, h] = L
    return out, lse
