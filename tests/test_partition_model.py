"""CPU model of the attention kernel's work partition: worker-wave shares, pool pieces and the
combine kernel's walk over their partials.

The kernel cuts a step's work blocks (per unit: UH virtual blocks, then its KV blocks) into
ranges with their own holder index, in work order: worker wave w's share [w*T1/W, (w+1)*T1/W),
then pool pieces [T1 + k*PS, T1 + (k+1)*PS) that finished waves claim in any order.  A range
splits at unit boundaries into segments; a segment that is not a whole unit leaves a partial in
its holder's slot 0 (the range's first segment) or 1, and the holder where a split unit starts
records the last holder of that unit: (U1*W - 1) / T1 for U1 <= T1, else W + (U1 - 1 - T1) / PS.
The combine walks holders h .. wb, slot `slot_a` for the first and 0 after.  This model checks,
on random batches and claim orders, that every KV block is computed exactly once and that each
split unit's walk finds exactly its partials, in block order.  It restates the partition rules
in Python; it is not the kernel's code.
"""

import random

import pytest


def _check_batch(seed, order_seed=0):
    rnd = random.Random(seed)
    BS = rnd.choice([16, 32])
    UH = rnd.choice([1, 2, 4, 12])
    Hkv, nrg = rnd.choice([1, 2, 8]), rnd.choice([1, 1, 2])
    lens = [rnd.choice([0, 1, rnd.randint(1, 200), rnd.randint(1, 6000)]) for _ in range(rnd.randint(1, 40))]
    units, off = [], 0                          # (first work block, KV blocks)
    for L in lens:
        nb = (L + BS - 1) // BS
        for _ in range(0 if L == 0 else Hkv * nrg):
            units.append((off, nb))
            off += UH + nb
    TB = off
    if TB == 0:
        return False
    PW = rnd.choice([3, 16, 48, 200, 768])     # worker waves launched
    W = min(PW, TB)
    pool_max = PW // 2 if rnd.random() < 0.8 else 0
    pct, PS = rnd.choice([5, 10, 20]), rnd.choice([1, 4, 12, 16])
    NP = min(pool_max, TB * pct // 100 // PS) if (pool_max > 0 and TB >= 32 * PW) else 0
    T1 = TB - NP * PS
    NH = PW + pool_max

    def unit_at(pos):
        for i, (u0, nb) in enumerate(units):
            if u0 <= pos < u0 + UH + nb:
                return i
        raise AssertionError(pos)

    covered, partials, whole, desc = {}, {}, set(), {}

    def run_holder(h, b0, b1):
        opened, pos, first = None, b0, True
        while pos < b1:
            ui = unit_at(pos)
            u0, nb = units[ui]
            uoff = pos - u0
            if uoff < UH:                        # virtual blocks: start at the unit's first KV block
                pos += UH - uoff
                continue
            ub = uoff - UH
            seg = min(nb - ub, b1 - pos)
            slot = 0 if first else 1
            for b in range(ub, ub + seg):
                assert (ui, b) not in covered
                covered[(ui, b)] = h
            if ub == 0 and seg == nb:
                whole.add(ui)
            else:
                assert (h, slot) not in partials
                partials[(h, slot)] = (ui, list(range(ub, ub + seg)))
                if ub == 0:
                    u1 = u0 + UH + nb
                    wb = (u1 * W - 1) // T1 if u1 <= T1 else W + (u1 - 1 - T1) // PS
                    opened = (ui, wb, slot)
            pos += seg
            first = False
        desc[h] = opened

    for w in range(W):
        run_holder(w, w * T1 // W, (w + 1) * T1 // W)
    if NP:
        assert W == PW                           # the pool follows the last share directly
    order = list(range(NP))
    random.Random(order_seed).shuffle(order)    # the order in which finished waves claim pieces
    for k in order:
        run_holder(W + k, T1 + k * PS, T1 + (k + 1) * PS)

    assert len(covered) == sum(nb for _, nb in units)
    used = set()
    for h, d in desc.items():
        if d is None:
            continue
        ui, wb, slot_a = d
        assert h < wb < NH
        got = []
        for wp in range(h, wb + 1):
            key = (wp, slot_a if wp == h else 0)
            assert key in partials and partials[key][0] == ui, (seed, key, d)
            got += partials[key][1]
            used.add(key)
        assert got == list(range(units[ui][1]))
    assert used == set(partials)
    return NP > 0


def test_partition_covers_every_block_once_and_the_combine_walk_finds_each_partial():
    with_pool = sum(_check_batch(seed) for seed in range(400))
    assert with_pool > 100                       # the pool is exercised, not only static shares


@pytest.mark.parametrize("order_seed", [1, 2, 3])
def test_any_claim_order_gives_the_same_decomposition_checks(order_seed):
    for seed in range(0, 400, 7):
        _check_batch(seed, order_seed)
