"""Seeded synthetic decode workloads shared by the tests, the smoke check and
the benchmark.

This module only draws inputs: sequence lengths, block tables built from a
shuffled list of physical ids, query / new-token / cache values, and NaN
poison in every pool slot that holds no token.  It holds none of the
attention or append arithmetic; both the oracle and the GPU library read the
arrays it produces.

Shapes follow the per-layer head shapes the pages use: a 13B-class model
(40 heads of 128) from [pofe] "The problem: reservation and fragmentation"
(OPT-13B), a 70B-class GQA model (8 KV heads of 128) from [arch] "KV Cache
Memory Bottlenecks", and the 32 query / 8 KV heads of 128 of the [arch]
"Production PyTorch Implementation" driver.  The pages measured on request
traces that are not available here; these seeded draws stand in for them.

Conventions
-----------
``lens[s]`` is the attention length L_s *after* the decode step's append.
The pool holds positions 0 .. L_s-2 of every sequence; position L_s-1 is the
token the step appends (from ``k_new`` / ``v_new``).  The table of sequence s
already lists ceil(L_s / B) blocks (the host has allocated the slot), and the
remaining entries are -1.  Every slot that holds no token before the append
(unallocated blocks, the tail of each sequence's last block, including the
append slot) is NaN when ``poison`` is set, so any read of it shows up in the
result.

FP8 pools (``kv_fp8=True``) hold E4M3FN codes drawn field by field: a random
sign, exponent field 3..10 and mantissa field 0..7 (magnitudes 2^-4 .. 15,
never NaN), with per-pool scales ``k_scale`` / ``v_scale``; empty slots hold
the NaN code 0x7F.  No quantisation is done here.  q and the new tokens keep
the config's 16-bit type.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

CONFIG_NAMES = {
    1: "tiny_fp32",
    2: "mha13b_bf16",
    3: "gqa70b_bf16",
    4: "shared_prefix_gqa_fp16",
    5: "long_context_gqa_bf16",
}


@dataclass
class Workload:
    name: str
    dtype: str
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    lens: np.ndarray                 # int32 [S], attention length after append
    tables: np.ndarray               # int32 [S, max_blocks], -1 padded
    q: torch.Tensor                  # [S, H_q, D]
    k_new: torch.Tensor              # [S, H_kv, D]
    v_new: torch.Tensor
    k_pool: torch.Tensor             # [N, B, H_kv, D], positions 0..L-2 filled
    v_pool: torch.Tensor
    partition_tokens: int = 512
    shared_blocks: list = field(default_factory=list)
    seed: int = 0
    kv_fp8: bool = False             # pools are torch.float8_e4m3fn codes
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return int(self.lens.shape[0])

    @property
    def lens_pre(self) -> np.ndarray:
        return (self.lens - 1).astype(np.int32)

    @property
    def max_blocks(self) -> int:
        return int(self.tables.shape[1])

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def default_seed(config_id: int) -> int:
    return 1000 + config_id


def _draw_lengths(config_id: int, rng: np.random.Generator, batch: int, len_range):
    lo, hi = len_range
    if config_id == 1:
        return np.array([10, 5, 13], dtype=np.int64)
    if config_id in (2, 5):
        return rng.integers(lo, hi + 1, size=batch)
    if config_id == 3:
        return np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch))).astype(np.int64)
    raise ValueError(config_id)


SPECS = {
    # id: dtype, B, H_q, H_kv, D, batch, length range
    1: ("f32", 4, 2, 1, 16, 3, (10, 13)),
    2: ("bf16", 16, 40, 40, 128, 64, (64, 2048)),
    3: ("bf16", 16, 64, 8, 128, 256, (512, 8192)),
    4: ("f16", 16, 32, 8, 128, 128, (1, 512)),       # suffix range; prefix 1024
    5: ("bf16", 16, 64, 8, 128, 8, (8192, 32768)),
}


def make_workload(config_id: int, seed: int | None = None, *, batch: int | None = None,
                  len_range=None, block_size: int | None = None, prefix_tokens: int = 1024,
                  device="cpu", poison: bool = True, dtype: str | None = None,
                  num_q_heads: int | None = None, num_kv_heads: int | None = None,
                  head_dim: int | None = None, shuffle: bool = True,
                  kv_fp8: bool = False) -> Workload:
    """Draw config ``config_id`` (1-5).  Keyword overrides shrink a config for
    tests while keeping its structure (length law, sharing, shuffled ids).
    ``shuffle=False`` hands out physical ids in order (identity-like tables)."""
    if seed is None:
        seed = default_seed(config_id)
    spec_dtype, spec_b, spec_hq, spec_hkv, spec_d, spec_batch, spec_range = SPECS[config_id]
    dtype = dtype or spec_dtype
    B = block_size or spec_b
    Hq = num_q_heads or spec_hq
    Hkv = num_kv_heads or spec_hkv
    D = head_dim or spec_d
    full_size = batch is None and len_range is None
    batch = batch or spec_batch
    len_range = len_range or spec_range
    rng = np.random.default_rng(seed)

    shared: list[int] = []
    if config_id == 4:
        suffix = rng.integers(len_range[0], len_range[1] + 1, size=batch)
        lens = prefix_tokens + suffix
        prefix_blocks = -(-prefix_tokens // B)
        if prefix_tokens % B != 0:
            raise ValueError("the shared prefix must fill whole blocks")
        private = [-(-int(L) // B) - prefix_blocks for L in lens]
        needed = prefix_blocks + sum(private)
        num_blocks = int(math.ceil(1.1 * needed)) + 128
    else:
        lens = _draw_lengths(config_id, rng, batch, len_range)
        nb = [-(-int(L) // B) for L in lens]
        if config_id == 1:
            num_blocks = 16
        elif config_id == 2 and full_size and B == 16:
            num_blocks = 16384
        else:
            num_blocks = int(math.ceil(1.1 * sum(nb))) + 1

    perm = rng.permutation(num_blocks) if shuffle else np.arange(num_blocks)
    nbs = [-(-int(L) // B) for L in lens]
    max_blocks = max(nbs)
    if config_id == 4 and full_size:
        max_blocks = 96
    elif config_id == 2 and full_size:
        max_blocks = 128
    elif config_id == 3 and full_size:
        max_blocks = 512
    elif config_id == 5 and full_size:
        max_blocks = 32768 // B
    elif config_id == 1:
        max_blocks = 4
    tables = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    pos = 0
    if config_id == 4:
        shared = [int(x) for x in perm[:prefix_blocks]]
        pos = prefix_blocks
        for s, n in enumerate(nbs):
            tables[s, :prefix_blocks] = shared
            k = n - prefix_blocks
            tables[s, prefix_blocks:n] = perm[pos:pos + k]
            pos += k
    else:
        for s, n in enumerate(nbs):
            tables[s, :n] = perm[pos:pos + n]
            pos += n
    used_ids = perm[:pos]
    unused_ids = perm[pos:]

    tdtype = DTYPES[dtype]
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    S = len(lens)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(tdtype)

    def codes(*shape):
        sign = torch.randint(0, 2, shape, generator=gen, device=dev, dtype=torch.int32)
        expo = torch.randint(3, 11, shape, generator=gen, device=dev, dtype=torch.int32)
        mant = torch.randint(0, 8, shape, generator=gen, device=dev, dtype=torch.int32)
        return ((sign << 7) | (expo << 3) | mant).to(torch.uint8).view(torch.float8_e4m3fn)

    q = randn(S, Hq, D)
    k_new = randn(S, Hkv, D)
    v_new = randn(S, Hkv, D)
    if kv_fp8:
        if dtype == "f32":
            raise ValueError("FP8 pools pair with 16-bit queries")
        k_pool = codes(num_blocks, B, Hkv, D)
        v_pool = codes(num_blocks, B, Hkv, D)
    else:
        k_pool = randn(num_blocks, B, Hkv, D)
        v_pool = randn(num_blocks, B, Hkv, D)
    if poison:
        # NaN, or for FP8 pools the NaN code 0x7F.
        nan = float("nan")
        if kv_fp8:
            k_pool = k_pool.view(torch.uint8)
            v_pool = v_pool.view(torch.uint8)
            nan = 0x7F
        if len(unused_ids):
            idx = torch.as_tensor(unused_ids, device=dev, dtype=torch.long)
            k_pool[idx] = nan
            v_pool[idx] = nan
        # The tail of each sequence's last block, from the append slot on,
        # holds no token yet.
        blk_idx, off_idx = [], []
        for s, (L, n) in enumerate(zip(lens, nbs)):
            last = int(tables[s, n - 1])
            first_empty = int(L) - 1 - (n - 1) * B
            for o in range(first_empty, B):
                blk_idx.append(last)
                off_idx.append(o)
        if blk_idx:
            bi = torch.as_tensor(blk_idx, device=dev, dtype=torch.long)
            oi = torch.as_tensor(off_idx, device=dev, dtype=torch.long)
            k_pool[bi, oi] = nan
            v_pool[bi, oi] = nan
        if kv_fp8:
            k_pool = k_pool.view(torch.float8_e4m3fn)
            v_pool = v_pool.view(torch.float8_e4m3fn)
    del used_ids
    return Workload(name=CONFIG_NAMES[config_id], dtype=dtype, block_size=B,
                    num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, num_blocks=num_blocks,
                    lens=lens.astype(np.int32), tables=tables, q=q, k_new=k_new, v_new=v_new,
                    k_pool=k_pool, v_pool=v_pool, shared_blocks=shared, seed=seed,
                    kv_fp8=kv_fp8, k_scale=0.0625 if kv_fp8 else 1.0,
                    v_scale=0.125 if kv_fp8 else 1.0)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a float32 / float16 / bfloat16 tensor to numpy float64."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def extract_sequences(w: Workload, seqs, dtype=np.float64):
    """Host float64 copies of the inputs of the chosen sequences only: the
    blocks their tables name (renumbered densely), their tables, lengths,
    queries and new tokens.  Lets a CPU reference run on a sample of a
    large GPU-resident workload."""
    seqs = [int(s) for s in seqs]
    nbs = [-(-int(w.lens[s]) // w.block_size) for s in seqs]
    ids = np.unique(np.concatenate([w.tables[s, :n] for s, n in zip(seqs, nbs)]))
    remap = {int(b): i for i, b in enumerate(ids)}
    idx = torch.as_tensor(ids, device=w.k_pool.device, dtype=torch.long)
    sel = torch.as_tensor(seqs, device=w.q.device, dtype=torch.long)
    tables = np.full((len(seqs), max(nbs)), -1, dtype=np.int64)
    for i, (s, n) in enumerate(zip(seqs, nbs)):
        tables[i, :n] = [remap[int(b)] for b in w.tables[s, :n]]
    def host(t):   # exact: every element type here widens exactly to float32/64
        return t.detach().to("cpu").to(torch.float64).numpy().astype(dtype)

    def pool(t):   # FP8 pools come back as their uint8 codes, undecoded
        if w.kv_fp8:
            return t.detach().view(torch.uint8).to("cpu").numpy().copy()
        return host(t)

    return dict(k_pool=pool(w.k_pool[idx]), v_pool=pool(w.v_pool[idx]), tables=tables,
                lens=w.lens[seqs].copy(), lens_pre=w.lens_pre[seqs].copy(),
                q=host(w.q[sel]), k_new=host(w.k_new[sel]), v_new=host(w.v_new[sel]))


# ---------------------------------------------------------------------------
# Prefill chunks
# ---------------------------------------------------------------------------

PREFILL_NAME = "prefill_gqa32x8_bf16"


@dataclass
class PrefillWorkload:
    """A packed prefill batch over a paged cache.

    Sequence s has ``lens[s]`` positions once its chunk is appended; the
    chunk is its last ``chunks[s]`` positions.  The pool holds positions
    0 .. lens[s] - chunks[s] - 1; the chunk's keys and values are in
    ``k_new`` / ``v_new`` (packed by ``cu``), its queries in ``q``.  Every
    other slot is NaN when poisoned.
    """
    name: str
    dtype: str
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    lens: np.ndarray        # int32 [S]
    chunks: np.ndarray      # int32 [S]
    cu: np.ndarray          # int32 [S + 1]
    tables: np.ndarray      # int32 [S, max_blocks], -1 padded
    q: torch.Tensor         # [T, H_q, D]
    k_new: torch.Tensor     # [T, H_kv, D]
    v_new: torch.Tensor
    k_pool: torch.Tensor    # [N, B, H_kv, D]
    v_pool: torch.Tensor
    seed: int = 0

    @property
    def lens_pre(self) -> np.ndarray:
        return (self.lens - self.chunks).astype(np.int32)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def make_prefill_workload(seed: int = 2000, *, batch: int = 16, lens=None, chunks=None,
                          block_size: int = 16, num_q_heads: int = 32, num_kv_heads: int = 8,
                          head_dim: int = 128, dtype: str = "bf16", device="cpu",
                          poison: bool = True, spare_blocks: int = 1) -> PrefillWorkload:
    """Draw a prefill batch.  Default: whole prompts (chunk = history) with the
    prompt-length law of the [pofe] "Simulation: batch size doubles,
    throughput does not" section (log-normal, median 584 and 95th percentile
    2,155 tokens, at most 4,096), on the 32 query / 8 KV heads of 128 of the
    [arch] "Production PyTorch Implementation" driver.  ``lens`` / ``chunks``
    override the draw (chunks default to the whole history)."""
    rng = np.random.default_rng(seed)
    if lens is None:
        sigma = math.log(2155 / 584) / 1.6448536269514722
        lens = np.rint(np.exp(rng.normal(math.log(584), sigma, size=batch)))
        lens = np.clip(lens, 16, 4096)
    lens = np.asarray(lens, dtype=np.int64)
    chunks = lens.copy() if chunks is None else np.asarray(chunks, dtype=np.int64)
    if chunks.shape != lens.shape or (chunks < 0).any() or (chunks > lens).any():
        raise ValueError("chunks must lie in [0, lens]")
    B = block_size
    nbs = [-(-int(L) // B) for L in lens]
    num_blocks = sum(nbs) + spare_blocks
    perm = rng.permutation(num_blocks)
    tables = np.full((len(lens), max(max(nbs), 1)), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(nbs):
        tables[s, :n] = perm[pos:pos + n]
        pos += n
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    T = int(cu[-1])

    tdtype = DTYPES[dtype]
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(tdtype)

    q = randn(T, num_q_heads, head_dim)
    k_new = randn(T, num_kv_heads, head_dim)
    v_new = randn(T, num_kv_heads, head_dim)
    k_pool = randn(num_blocks, B, num_kv_heads, head_dim)
    v_pool = randn(num_blocks, B, num_kv_heads, head_dim)
    if poison:
        empty = np.ones((num_blocks, B), dtype=bool)     # slots holding no token yet
        for s, n in enumerate(nbs):
            held = int(lens[s] - chunks[s])
            for t in range(held):
                empty[tables[s, t // B], t % B] = False
        mask = torch.as_tensor(empty, device=dev)
        k_pool[mask] = float("nan")
        v_pool[mask] = float("nan")
    return PrefillWorkload(name=PREFILL_NAME, dtype=dtype, block_size=B,
                           num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                           head_dim=head_dim, num_blocks=num_blocks,
                           lens=lens.astype(np.int32), chunks=chunks.astype(np.int32), cu=cu,
                           tables=tables, q=q, k_new=k_new, v_new=v_new, k_pool=k_pool,
                           v_pool=v_pool, seed=seed)
