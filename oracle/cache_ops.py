"""Cache append and block copy on copies of the pools (oracle).

Test infrastructure only; see the package docstring for who may use it.
Both operations are byte moves, so the result is exact and a GPU result must
match it bit for bit.
"""

from __future__ import annotations

import numpy as np

from .paging import resolve


def append_token(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
                 v_new: np.ndarray, tables: np.ndarray, lens_pre, block_size: int):
    """Write each sequence's new token into its slot; return new pools.

    [pofe] "How it works", decode step: the new token's k and v go to slot
    len mod b of the last table entry, where len is the length before the
    append ([pofe] "Minimal implementation", ``Sequence.append`` writes at
    ``self.len % b`` and then increments ``len``).  Resolving position len
    through the table names that same block (floor(len / b) is the last
    entry once the host has allocated it).  A negative length marks a padding
    row that writes nothing.  Every other byte of the pools is unchanged.

    k_new, v_new: [S, H_kv, D]; pools: [N, B, H_kv, D]; lens_pre: [S].
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    num_blocks = k_pool.shape[0]
    for s, length in enumerate(lens_pre):
        length = int(length)
        if length < 0:
            continue
        physical, offset = resolve(tables[s], block_size, length)
        if not (0 <= physical < num_blocks):
            raise IndexError(f"sequence {s}: block id {physical} outside the pool")
        k_out[physical, offset] = k_new[s]
        v_out[physical, offset] = v_new[s]
    return k_out, v_out


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, src, dst):
    """Copy whole blocks (all B slots, all heads) src[i] -> dst[i]; return new pools.

    The copy-on-write step of [arch] 4. ("copy the B tokens from the shared
    block to the new block") and [pofe] "Minimal implementation"
    (``p.k[:, new] = p.k[:, old]``).  The destinations must be distinct and
    must not also be sources, so the order of the copies does not matter.
    """
    src = [int(x) for x in src]
    dst = [int(x) for x in dst]
    if len(set(dst)) != len(dst) or set(dst) & set(src):
        raise ValueError("destinations must be distinct and disjoint from sources")
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for a, b in zip(src, dst):
        k_out[b] = k_pool[a]
        v_out[b] = v_pool[a]
    return k_out, v_out


def append_tokens(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
                  v_new: np.ndarray, tables: np.ndarray, lens_pre, cu_seqlens,
                  block_size: int):
    """Write a run of new tokens per sequence into its slots; return new pools.

    The multi-token form of :func:`append_token`: sequence s appends the
    n_s = cu_seqlens[s+1] - cu_seqlens[s] rows k_new[cu_seqlens[s] + j],
    j < n_s, at positions lens_pre[s] + j, each resolved through the table
    ([pofe] "How it works": the prompt's blocks are allocated at admission
    and prefill writes into them; slot p mod b of entry floor(p / b)).  A
    negative lens_pre marks a padding row that writes nothing.

    k_new, v_new: [T, H_kv, D] packed; pools [N, B, H_kv, D]; lens_pre [S];
    cu_seqlens [S + 1].
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    num_blocks = k_pool.shape[0]
    cu = [int(x) for x in cu_seqlens]
    for s, start in enumerate(lens_pre):
        start = int(start)
        if start < 0:
            continue
        for j in range(cu[s + 1] - cu[s]):
            physical, offset = resolve(tables[s], block_size, start + j)
            if not (0 <= physical < num_blocks):
                raise IndexError(f"sequence {s}: block id {physical} outside the pool")
            k_out[physical, offset] = k_new[cu[s] + j]
            v_out[physical, offset] = v_new[cu[s] + j]
    return k_out, v_out


def swap_out(k_pool: np.ndarray, v_pool: np.ndarray, ids):
    """Copy whole blocks ids[i] to host buffers slot i; return (host_k, host_v).

    [pofe] "When memory runs out": a preempted sequence's blocks are copied
    to CPU memory and back later; [lesson] "Preemption": copy blocks to
    pinned host memory and back.  The host buffers are [n, B, H_kv, D]; slot
    i holds block ids[i] bit for bit.
    """
    ids = [int(x) for x in ids]
    num_blocks = k_pool.shape[0]
    if any(not (0 <= i < num_blocks) for i in ids):
        raise IndexError("block id outside the pool")
    return k_pool[ids].copy(), v_pool[ids].copy()


def swap_in(k_pool: np.ndarray, v_pool: np.ndarray, ids, host_k: np.ndarray,
            host_v: np.ndarray):
    """Copy host slot i back into block ids[i]; return new pools.  The ids
    must be distinct (each names the block a swapped-in sequence now owns)."""
    ids = [int(x) for x in ids]
    num_blocks = k_pool.shape[0]
    if len(set(ids)) != len(ids):
        raise ValueError("swap-in destinations must be distinct")
    if any(not (0 <= i < num_blocks) for i in ids):
        raise IndexError("block id outside the pool")
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for slot, i in enumerate(ids):
        k_out[i] = host_k[slot]
        v_out[i] = host_v[slot]
    return k_out, v_out
