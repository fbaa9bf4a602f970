"""Decode attention over a paged KV cache, in float64 (oracle).

Test infrastructure only; see the package docstring for who may use it.

The method reaches exactly the ordinary attention result: [pofe] "How it
works" says the math is unchanged and only the addresses are indirect, and
[note] "The kernel must understand the mapping" says paging does not change
the softmax distribution.  So the reference here is the plain definition,
computed on an explicit contiguous copy made through the block table:

    o_h = sum_t softmax_t(scale * q_h . K[t, kvh(h)]) * V[t, kvh(h)]

with kvh(h) = floor(h / g), g = H_q / H_kv ([pofe] "Minimal implementation":
``repeat_interleave`` of the KV heads; [arch] Step 2, the grouped-query
ratio) and scale = 1 / sqrt(head_dim) by default ([arch] 3. Non-Contiguous
Online Softmax Attention Kernel, standard attention with sqrt(d_k)).

Two further functions restate the block-wise online-softmax recurrence of
[arch] 3. and the merge of partial softmax states (the operator that
combines per-block terms in the same section), so that tests can check that
both reach the two-pass result.
"""

from __future__ import annotations

import math

import numpy as np

from .paging import gather_contiguous, blocks_needed


def _softmax_weights(z: np.ndarray) -> np.ndarray:
    """Two-pass stable softmax over the last axis: exp(z - max z) / sum."""
    shifted = z - z.max(axis=-1, keepdims=True)
    e = np.exp(shifted)
    return e / e.sum(axis=-1, keepdims=True)


def decode_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                     tables: np.ndarray, lens, block_size: int,
                     scale: float | None = None) -> np.ndarray:
    """Paged decode attention for a batch of sequences, one query token each.

    q:       [S, H_q, D]
    k_pool:  [N, B, H_kv, D]   (v_pool the same)
    tables:  [S, max_blocks]   physical ids; entries past ceil(L_s/B) unused
    lens:    [S]               attention length L_s of each sequence
    returns  float64 [S, H_q, D]; a sequence with L_s = 0 gets zeros (the
             [arch] Step 2 function leaves such rows at their zero init).
    """
    q = np.asarray(q, dtype=np.float64)
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = k_pool.shape[2]
    if num_q_heads % num_kv_heads != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = num_q_heads // num_kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        length = int(lens[s])
        if length == 0:
            continue
        k_seq = gather_contiguous(k_pool, tables[s], length, block_size).astype(np.float64)
        v_seq = gather_contiguous(v_pool, tables[s], length, block_size).astype(np.float64)
        for h in range(num_q_heads):
            kvh = h // group
            z = scale * (k_seq[:, kvh, :] @ q[s, h])          # [L]
            p = _softmax_weights(z)                            # [L]
            out[s, h] = p @ v_seq[:, kvh, :]                   # [D]
    return out


# ---------------------------------------------------------------------------
# Block-wise online softmax and the merge of partial states
# ---------------------------------------------------------------------------

def online_softmax_blocks(q_h: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                          table_row, length: int, block_size: int, kv_head: int,
                          scale: float, first_block: int = 0,
                          last_block: int | None = None):
    """Run the [arch] 3. recurrence over logical blocks [first, last).

    For each block b: S_b = scale * q K_b^T with tail positions (t >= length)
    masked to -inf (the mask term M_b); m_new = max(m, max_j S_b,j);
    P_b = exp(S_b - m_new); l = l * exp(m - m_new) + sum_j P_b,j;
    o = o * exp(m - m_new) + P_b V_b.  Returns the unnormalised state
    (m, l, o); the page's final output is o / l.
    """
    q_h = np.asarray(q_h, dtype=np.float64)
    if last_block is None:
        last_block = blocks_needed(length, block_size)
    m = -math.inf
    l = 0.0
    o = np.zeros(q_h.shape[0], dtype=np.float64)
    for b in range(first_block, last_block):
        physical = int(table_row[b])
        k_blk = k_pool[physical, :, kv_head, :].astype(np.float64)   # [B, D]
        v_blk = v_pool[physical, :, kv_head, :].astype(np.float64)
        positions = b * block_size + np.arange(block_size)
        valid = positions < length
        s_b = np.full(block_size, -math.inf)
        s_b[valid] = scale * (k_blk[valid] @ q_h)
        m_new = max(m, s_b.max())
        p_b = np.zeros(block_size)
        p_b[valid] = np.exp(s_b[valid] - m_new)
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        l = l * alpha + p_b.sum()
        o = o * alpha + p_b[valid] @ v_blk[valid]
        m = m_new
    return m, l, o


def merge_states(states):
    """Combine partial softmax states (m_p, l_p, o_p) of disjoint token sets.

    With M = max_p m_p:  O = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p.
    This is the block-combining operator of [arch] 3. applied to groups of
    blocks instead of single blocks.  Empty states (m = -inf) contribute 0.
    Returns the normalised output (zeros if every state is empty).
    """
    finite = [st for st in states if st[0] != -math.inf]
    if not finite:
        d = states[0][2].shape[0] if states else 0
        return np.zeros(d)
    big_m = max(st[0] for st in finite)
    num = sum(math.exp(m - big_m) * o for m, _, o in finite)
    den = sum(math.exp(m - big_m) * l for m, l, _ in finite)
    return num / den


def split_k_decode_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                             tables: np.ndarray, lens, block_size: int,
                             partition_tokens: int, scale: float | None = None) -> np.ndarray:
    """Decode attention computed as partitions of ``partition_tokens`` tokens,
    each run through the online recurrence, then merged with
    :func:`merge_states`.  Mathematically equal to :func:`decode_attention`."""
    q = np.asarray(q, dtype=np.float64)
    num_seqs, num_q_heads, head_dim = q.shape
    group = num_q_heads // k_pool.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    if partition_tokens % block_size != 0:
        raise ValueError("partition_tokens must be a multiple of block_size")
    blocks_per_part = partition_tokens // block_size
    out = np.zeros((num_seqs, num_q_heads, head_dim))
    for s in range(num_seqs):
        length = int(lens[s])
        if length == 0:
            continue
        nb = blocks_needed(length, block_size)
        for h in range(num_q_heads):
            states = []
            for first in range(0, nb, blocks_per_part):
                last = min(first + blocks_per_part, nb)
                states.append(online_softmax_blocks(q[s, h], k_pool, v_pool, tables[s],
                                                    length, block_size, h // group,
                                                    scale, first, last))
            out[s, h] = merge_states(states)
    return out


# ---------------------------------------------------------------------------
# Chunked prefill over the paged cache
# ---------------------------------------------------------------------------

def prefill_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                      tables: np.ndarray, lens, cu_seqlens, block_size: int,
                      scale: float | None = None) -> np.ndarray:
    """Causal attention of a chunk of query tokens per sequence over its
    paged history.

    [pofe] "How it works": at admission the prompt's blocks are allocated
    and prefill writes into them, and attention over a block table is the
    ordinary attention sum (one row of weights per query i) regrouped by
    block; [pofe] "When memory runs out" and [lesson] "Preemption": a
    recomputed sequence is prefilled again from its tokens in one pass.
    The pages do not spell out the mask.  Reading: each query token attends
    to itself and every earlier position, the decode rule applied to every
    token of the chunk.  Sequence s holds L_s = lens[s] positions (the
    chunk's own keys and values already appended), and its chunk is its last
    n_s = cu_seqlens[s+1] - cu_seqlens[s] positions, so query j of the chunk
    sits at position p = L_s - n_s + j and attends positions 0 .. p:

        o[j, h] = sum_{t <= p} softmax_t(scale * q[j, h] . K[t, kvh(h)]) V[t, kvh(h)]

    q:          [T, H_q, D], T = cu_seqlens[-1] (the chunks, packed)
    pools:      [N, B, H_kv, D]; tables [S, max_blocks]
    lens:       [S] context lengths including the chunk (n_s <= L_s)
    cu_seqlens: [S + 1] chunk offsets into q, non-decreasing from 0
    returns     float64 [T, H_q, D]
    """
    q = np.asarray(q, dtype=np.float64)
    total, num_q_heads, head_dim = q.shape
    num_kv_heads = k_pool.shape[2]
    if num_q_heads % num_kv_heads != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = num_q_heads // num_kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    cu = [int(x) for x in cu_seqlens]
    if cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must rise from 0 to the number of query tokens")
    out = np.zeros((total, num_q_heads, head_dim), dtype=np.float64)
    for s in range(len(cu) - 1):
        n = cu[s + 1] - cu[s]
        length = int(lens[s])
        if n == 0:
            continue
        if n > length:
            raise ValueError(f"sequence {s}: chunk of {n} tokens exceeds its length {length}")
        k_seq = gather_contiguous(k_pool, tables[s], length, block_size).astype(np.float64)
        v_seq = gather_contiguous(v_pool, tables[s], length, block_size).astype(np.float64)
        for j in range(n):
            pos = length - n + j
            for h in range(num_q_heads):
                kvh = h // group
                z = scale * (k_seq[: pos + 1, kvh, :] @ q[cu[s] + j, h])   # [pos + 1]
                p = _softmax_weights(z)
                out[cu[s] + j, h] = p @ v_seq[: pos + 1, kvh, :]
    return out


def decode_log_normaliser(q: np.ndarray, k_pool: np.ndarray, tables: np.ndarray, lens,
                          block_size: int, scale: float | None = None) -> np.ndarray:
    """Natural log of each head's softmax normaliser in decode attention:
    lse[s, h] = ln sum_{t<L_s} exp(scale * q[s, h] . K[t, kvh(h)]), computed as
    max z + ln sum exp(z - max z) (the stabilising shift of the two-pass
    softmax above).  -inf for an empty sequence.  Two normalised partial
    results over disjoint key sets combine with these weights, which is how
    the merge of [arch] 3. reads when each part is already normalised."""
    q = np.asarray(q, dtype=np.float64)
    num_seqs, num_q_heads, head_dim = q.shape
    group = num_q_heads // k_pool.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    out = np.full((num_seqs, num_q_heads), -math.inf)
    for s in range(num_seqs):
        length = int(lens[s])
        if length == 0:
            continue
        k_seq = gather_contiguous(k_pool, tables[s], length, block_size).astype(np.float64)
        for h in range(num_q_heads):
            z = scale * (k_seq[:, h // group, :] @ q[s, h])
            zmax = z.max()
            out[s, h] = zmax + math.log(np.exp(z - zmax).sum())
    return out
