"""The seeded generators draw the configs they claim to draw.

The NaN poison must cover exactly the slots that hold no token before the
append: this is checked against the oracle's own block-table resolution.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import paging


def finite_slots(pool):
    return torch.isfinite(pool.float()).all(dim=-1).all(dim=-1).numpy()


@pytest.mark.parametrize("cid,kw", [
    (1, {}),
    (2, dict(batch=5, len_range=(1, 70))),
    (3, dict(batch=6, len_range=(17, 300))),
    (4, dict(batch=4, len_range=(1, 40), prefix_tokens=64)),
    (5, dict(batch=3, len_range=(100, 400), block_size=8)),
    (5, dict(batch=3, len_range=(100, 400), block_size=32)),
])
def test_poison_covers_exactly_the_empty_slots(cid, kw):
    w = workloads.make_workload(cid, **kw)
    mask = paging.valid_slot_mask(w.tables, w.lens_pre, w.num_blocks, w.block_size)
    assert (finite_slots(w.k_pool) == mask).all()
    assert (finite_slots(w.v_pool) == mask).all()
    for s, L in enumerate(w.lens):
        nb = paging.blocks_needed(int(L), w.block_size)
        assert (w.tables[s, :nb] >= 0).all() and (w.tables[s, nb:] == -1).all()
        assert (w.tables[s, :nb] < w.num_blocks).all()


def test_tiny_config_shape():
    w = workloads.make_workload(1)
    assert list(w.lens) == [10, 5, 13]
    assert w.num_blocks == 16 and w.block_size == 4 and w.dtype == "f32"
    used = w.tables[w.tables >= 0]
    assert len(used) == 9 and len(set(used.tolist())) == 9
    assert w.q.shape == (3, 2, 16) and w.k_pool.shape == (16, 4, 1, 16)
    # Appends land at offsets 1, 0, 0 (9, 4 and 12 mod 4): a write into a
    # partly filled block and two into fresh blocks.
    assert [int(L - 1) % 4 for L in w.lens] == [1, 0, 0]


def test_shared_prefix_structure():
    w = workloads.make_workload(4, batch=6, len_range=(1, 40), prefix_tokens=64)
    assert w.dtype == "f16"
    pb = 64 // 16
    assert (w.tables[:, :pb] == np.array(w.shared_blocks)).all()
    private = w.tables[:, pb:]
    private = private[private >= 0]
    assert len(set(private.tolist())) == len(private)
    assert not set(private.tolist()) & set(w.shared_blocks)


def test_full_size_structures():
    # Structure only (small value tensors are drawn, but the lengths and
    # tables follow the full configs): pool sizes and table widths.
    rng = np.random.default_rng(workloads.default_seed(3))
    w3 = workloads.make_workload(3, batch=256, len_range=(512, 8192), head_dim=8,
                                 num_q_heads=8, num_kv_heads=1, poison=False)
    assert w3.lens.min() >= 512 and w3.lens.max() <= 8192
    nb = sum(paging.blocks_needed(int(L), 16) for L in w3.lens)
    assert w3.num_blocks == int(np.ceil(1.1 * nb)) + 1
    del rng


def test_seeded_repeatable():
    a = workloads.make_workload(2, batch=3, len_range=(5, 50))
    b = workloads.make_workload(2, batch=3, len_range=(5, 50))
    assert np.array_equal(a.tables, b.tables)
    assert torch.equal(a.q, b.q)
    assert torch.equal(a.k_pool.isnan(), b.k_pool.isnan())
