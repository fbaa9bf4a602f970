"""Contiguous reservation vs paged on-demand allocation of a toy workload.

Test infrastructure only; see the package docstring for who may use it.

[lesson] "Developer — The allocator, both strategies" runs four requests,
each a (prompt tokens, generated tokens) pair, through two allocators on a
pool of 64 blocks of 16 slots and prints what each one holds.  The functions
here recompute those quantities: the contiguous one in closed form from the
reservation rule (not by replaying the page's loop), the paged one by driving :class:`oracle.block_manager.OracleSequence`
(prompt blocks at admission, one more block whenever the last fills), so that
the page's printed numbers pin the block manager's allocation rule.
"""

from __future__ import annotations

from .block_manager import NoFreeBlock, OracleBlockPool, OracleSequence


def contiguous_reservation(requests: dict, pool_slots: int, max_len: int) -> dict:
    """Reservation rule: every request asks for the same ``max_len`` slots, so
    in arrival order the first ``pool_slots // max_len`` requests fit and the
    rest are turned away.  A served request wastes ``max_len`` minus the
    tokens it ends up holding (prompt + generated); the pool's waste is the
    share of the reserved slots that hold no token.  Returns per-request
    (reserved, used, wasted), or the free slots a rejected request found, and
    the totals."""
    names = list(requests)
    admitted = names[:min(len(names), pool_slots // max_len)]
    reserved = len(admitted) * max_len
    used = {n: requests[n][0] + requests[n][1] for n in names}
    per_request = {}
    for n in names:
        if n in admitted:
            per_request[n] = {"reserved": max_len, "used": used[n], "wasted": max_len - used[n]}
        else:
            per_request[n] = {"rejected": True, "free_slots": pool_slots - reserved}
    needed = sum(used[n] for n in admitted)
    waste_pct = 100.0 * (1.0 - needed / reserved) if reserved else 0.0
    return {"per_request": per_request, "served": len(admitted), "reserved": reserved,
            "needed": needed, "waste_pct": waste_pct}


def paged_on_demand(requests: dict, pool_blocks: int, block_size: int) -> dict:
    """Admit each prompt with ceil(p / B) blocks, then decode its generated
    tokens one at a time, taking a block only when the last one is full."""
    pool = OracleBlockPool(pool_blocks, block_size)
    per_request = {}
    held_blocks = 0
    for name, (prompt, gen) in requests.items():
        seq = OracleSequence(pool)
        try:
            seq.reserve_prompt(prompt)
        except NoFreeBlock:
            per_request[name] = {"rejected": True}
            continue
        preempted = False
        for _ in range(gen):
            try:
                seq.append_slot()
            except NoFreeBlock:
                preempted = True
                break
        blocks = len(seq.table)
        held_blocks += blocks
        per_request[name] = {"blocks": blocks, "tokens": seq.len,
                             "wasted": blocks * block_size - seq.len,
                             "preempted": preempted}
    held = held_blocks * block_size
    needed = sum(p + g for p, g in requests.values())
    served = sum(1 for r in per_request.values() if not r.get("rejected"))
    return {"per_request": per_request, "served": served, "held": held, "needed": needed,
            "waste_pct": 100.0 * (held - needed) / held if held else 0.0,
            "free_blocks": pool.num_free()}


def shared_prompt(sys_tokens: int, users: int, block_size: int) -> dict:
    """One system prompt used by ``users`` sequences: blocks if each user
    holds a private copy vs one shared copy with a reference count per block
    ([lesson] "The second gift: sharing"; the toy's last section)."""
    pool = OracleBlockPool(users * (-(-sys_tokens // block_size)) + 1, block_size)
    first = OracleSequence(pool)
    first.reserve_prompt(sys_tokens)
    others = [first.fork() for _ in range(users - 1)]
    shared_blocks = len(first.table)
    refcount = pool.ref[first.table[0]]
    copied = users * shared_blocks
    saved_slots = (copied - shared_blocks) * block_size
    for s in [first] + others:
        s.free_all()
    return {"copied_blocks": copied, "shared_blocks": shared_blocks,
            "refcount": refcount, "saved_slots": saved_slots,
            "all_free_after": pool.num_free() == pool.num_blocks}
