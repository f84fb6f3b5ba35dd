"""Pins for the oracle's moe_align (block-aligned routing buffers).

The oracle's answer is checked against the properties that determine it
uniquely (brute force over every tiny input), against closed forms, and
against a hand-worked example under tests/golden/.
"""
import itertools
import os

import numpy as np
import pytest

from oracle import qma_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_align_properties(ids, E, B, sorted_ids, expert_ids, ntp, cap):
    """Every property the buffers must have. Together they fix the result."""
    ids = np.asarray(ids).reshape(-1)
    R = ids.size
    ntp = int(ntp)
    blocks_cap = -(-cap // B)
    assert sorted_ids.shape == (cap,) and expert_ids.shape == (blocks_cap,)
    assert ntp % B == 0 and 0 <= ntp <= cap
    # tails
    assert np.all(sorted_ids[ntp:] == R)
    assert np.all(expert_ids[ntp // B:] == -1)
    # every valid slot exactly once, invalid slots never
    body = sorted_ids[:ntp]
    real = body[body != R]
    valid = [i for i in range(R) if 0 <= ids[i] < E]
    assert sorted(real.tolist()) == valid
    # each block's slots belong to its expert
    prev_e = -1
    for b in range(ntp // B):
        e = int(expert_ids[b])
        assert 0 <= e < E and e >= prev_e
        seg = sorted_ids[b * B:(b + 1) * B]
        for s in seg:
            assert s == R or ids[s] == e
        prev_e = e
    # per expert: contiguous blocks, ascending slots first then sentinels,
    # block count ceil(c_e / B), zero-count experts get none
    for e in range(E):
        blocks = [b for b in range(ntp // B) if expert_ids[b] == e]
        c = int(np.sum(ids == e))
        assert len(blocks) == -(-c // B)
        if blocks:
            assert blocks == list(range(blocks[0], blocks[0] + len(blocks)))
            seg = sorted_ids[blocks[0] * B:(blocks[-1] + 1) * B].tolist()
            assert seg[:c] == sorted(seg[:c]) and all(s != R for s in seg[:c])
            assert all(s == R for s in seg[c:])


def test_brute_force_all_tiny_routings():
    n = 0
    for T, topk, E in [(1, 1, 1), (2, 1, 3), (3, 1, 2), (2, 2, 3), (3, 2, 2),
                       (3, 2, 3)]:
        for combo in itertools.product(range(-1, E), repeat=T * topk):
            ids = np.array(combo, dtype=np.int32).reshape(T, topk)
            for B in (1, 2, 4):
                cap, _ = O.align_sizes(T, topk, E, B)
                s, e, ntp = O.moe_align(ids, E, B)
                check_align_properties(ids, E, B, s, e, ntp, cap)
                s2, e2, ntp2 = O.moe_align_fast(ids, E, B)
                assert np.array_equal(s, s2) and np.array_equal(e, e2)
                assert ntp == ntp2
                n += 1
    assert n > 3000


def test_hand_worked_golden():
    d = {}
    with open(os.path.join(GOLDEN, "moe_align_hand.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, *v = line.split()
                d[k] = [int(x) for x in v]
    T, topk, E, B = d["T"][0], d["topk"][0], d["E"][0], d["block_m"][0]
    ids = np.array(d["topk_ids"], dtype=np.int32).reshape(T, topk)
    s, e, ntp = O.moe_align(ids, E, B)
    assert s.tolist() == d["sorted_ids"]
    assert e.tolist() == d["expert_ids"]
    assert int(ntp) == d["num_tokens_padded"][0]


def test_closed_form_all_on_one_expert():
    T, topk, E, B = 5, 2, 4, 4
    ids = np.full((T, topk), 2, dtype=np.int32)
    s, e, ntp = O.moe_align(ids, E, B)
    R = T * topk
    assert int(ntp) == 12
    assert s[:R].tolist() == list(range(R)) and np.all(s[R:] == R)
    assert e[:3].tolist() == [2, 2, 2] and np.all(e[3:] == -1)


def test_closed_form_one_slot_per_expert():
    E, B = 6, 4
    ids = np.random.default_rng(0).permutation(E).astype(np.int32)[:, None]
    s, e, ntp = O.moe_align(ids, E, B)
    assert int(ntp) == E * B
    for b in range(E):
        assert s[b * B] == int(np.nonzero(ids[:, 0] == b)[0][0])
        assert np.all(s[b * B + 1:(b + 1) * B] == E)
        assert e[b] == b


def test_many_empty_experts():
    E, B = 384, 16
    ids = np.array([[5], [300], [5]], dtype=np.int32)
    s, e, ntp = O.moe_align(ids, E, B)
    assert int(ntp) == 32 and e[:2].tolist() == [5, 300]
    assert s[:3].tolist() == [0, 2, 3] and s[16] == 1


@pytest.mark.parametrize("seed", range(6))
def test_fast_matches_plain_random(seed):
    rng = np.random.default_rng(seed)
    T, topk, E = int(rng.integers(1, 300)), int(rng.integers(1, 9)), int(rng.integers(1, 70))
    B = int(rng.choice([1, 16, 32, 64, 128]))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    cap, _ = O.align_sizes(T, topk, E, B)
    extra = int(rng.integers(0, 3 * B))                 # over-allocated buffers
    a = O.moe_align(ids, E, B, cap + extra)
    b = O.moe_align_fast(ids, E, B, cap + extra)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert a[2] == b[2]
    check_align_properties(ids, E, B, *a, cap + extra)


def test_capacity_bound_is_tight_enough():
    # worst case: every expert has count = 1 mod B
    E, B = 7, 8
    ids = np.repeat(np.arange(E), 9)[:, None].astype(np.int32)
    cap, _ = O.align_sizes(ids.shape[0], 1, E, B)
    s, e, ntp = O.moe_align(ids, E, B, cap)
    assert int(ntp) == E * 16 and int(ntp) <= cap
