"""Block-table resolution, explicit gather and slot accounting (oracle).

Test infrastructure only; see the package docstring for who may use it.

Pool layout read here: ``pool[num_blocks, block_size, num_kv_heads, head_dim]``,
the per-layer cache tensor shape of [arch] "Production PyTorch Implementation",
Step 2 (the ``k_cache`` / ``v_cache`` arguments), which is also the
per-layer slice of [pofe] "Minimal implementation" (``BlockPool.k``).
"""

from __future__ import annotations

import numpy as np


def resolve(table_row, block_size: int, t: int) -> tuple[int, int]:
    """Map token position ``t`` of one sequence to (physical block id, offset).

    [arch] "Mathematical Foundations", 1. Paged Virtual Memory Mapping: the
    logical block index is floor(t / B), the offset inside it is t mod B, and
    the block table maps the logical index to a physical block id.
    [note] "Map a ten-token sequence into pages" works the same mapping by hand.
    """
    if t < 0:
        raise ValueError("token position must be non-negative")
    logical = t // block_size
    offset = t % block_size
    return int(table_row[logical]), offset


def element_offset(physical: int, offset: int, kv_head: int, d: int,
                   block_size: int, num_kv_heads: int, head_dim: int) -> int:
    """Element index of ``pool[physical, offset, kv_head, d]`` in a flat pool.

    The address formula of [arch] 1. Paged Virtual Memory Mapping gives
    block stride B * H_kv * d_head and token stride d_head but mixes bytes
    with elements and leaves out the head term; this is the reading that
    matches the [N, B, H_kv, D] tensors the same page allocates (row-major).
    """
    return ((physical * block_size + offset) * num_kv_heads + kv_head) * head_dim + d


def blocks_needed(n_tokens: int, block_size: int) -> int:
    """ceil(n / B): [arch] 1. Paged Virtual Memory Mapping ("partitioned into
    ceil(s/B) logical blocks")."""
    return -(-n_tokens // block_size)


def slots_allocated(n_tokens: int, block_size: int) -> int:
    """B * ceil(n / B): [note] "Quantify the remaining internal fragmentation"."""
    return block_size * blocks_needed(n_tokens, block_size)


def wasted_slots(n_tokens: int, block_size: int) -> int:
    """Allocated minus used slots, in [0, B-1]: [note] same section;
    [arch] 2. Memory Utilization Bound ("Wasted Slots")."""
    return slots_allocated(n_tokens, block_size) - n_tokens


def eta_paged(s: int, block_size: int) -> float:
    """Utilisation s / (ceil(s/B) * B): [arch] 2. Memory Utilization Bound."""
    return s / slots_allocated(s, block_size)


def eta_paged_lower_bound(s: int, block_size: int) -> float:
    """The page's lower bound s / (s + B) = 1 - B / (s + B)."""
    return 1.0 - block_size / (s + block_size)


def eta_naive(s: int, l_max: int) -> float:
    """Utilisation of a contiguous reservation of L_max slots: s / L_max."""
    return s / l_max


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       dtype_bytes: int) -> int:
    """M_KV(s) / s = 2 * N_layers * N_kv * d_head * sizeof:
    [arch] "KV Cache Memory Bottlenecks in Autoregressive Serving"."""
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def gather_contiguous(pool: np.ndarray, table_row, length: int,
                      block_size: int) -> np.ndarray:
    """Materialise the contiguous [length, H_kv, D] history of one sequence.

    This is the explicit gather of [pofe] "Minimal implementation" (index the
    pool by the table, flatten blocks x slots, keep the first ``len`` rows),
    done one token at a time through :func:`resolve` so that every position
    visibly goes through the table.  Block ids outside [0, num_blocks) are an
    error ([note] "Useful allocator invariants": every live logical block must
    refer to valid physical storage).
    """
    num_blocks = pool.shape[0]
    out = np.empty((length,) + pool.shape[2:], dtype=pool.dtype)
    for t in range(length):
        physical, offset = resolve(table_row, block_size, t)
        if not (0 <= physical < num_blocks):
            raise IndexError(f"token {t}: block id {physical} outside [0, {num_blocks})")
        out[t] = pool[physical, offset]
    return out


def valid_slot_mask(tables: np.ndarray, lens, num_blocks: int,
                    block_size: int) -> np.ndarray:
    """Boolean [num_blocks, B]: True where some sequence holds a token.

    Used by tests to check that data outside the valid slots is never read.
    """
    mask = np.zeros((num_blocks, block_size), dtype=bool)
    for s, length in enumerate(lens):
        for t in range(int(length)):
            physical, offset = resolve(tables[s], block_size, t)
            mask[physical, offset] = True
    return mask


def utilisation_paged_worst(mean_len: float, block_size: int) -> float:
    """Batch utilisation when every sequence wastes the most it can, B - 1
    slots: mean / (mean + B - 1).  [pofe] "The memory accounting" states the
    bound (its formula is missing from the extracted text; this is the
    reading that reproduces the page's 98.5 % at mean 1000, B = 16)."""
    return mean_len / (mean_len + block_size - 1)


def utilisation_reserve(mean_len: float, s_max: int) -> float:
    """Utilisation under per-request reservation of S_max: mean / S_max."""
    return mean_len / s_max

