"""Pins of the oracle's host block pool (reading R12 for the hand-out order). CPU only.

Pins: the page's worked allocation (68 tokens, block_size 32 -> 3 blocks),
invariants checked by brute force over random steps and releases (every block
owned once, ceil(len / bs) blocks per sequence, every live position's slot
unique and decoding to its table entry and offset), an out-of-space step that
changes nothing, the stated hand-out order on a hand-worked case, and paged ==
dense attention when keys and values go in through the pool's slots and come
back through its tables."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.block_pool import BlockPool, NoSpace

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")


def test_page_example_68_tokens_in_blocks_of_32():
    ex = json.load(open(GOLDEN))["block_allocation"]
    pool = BlockPool(num_blocks=8, block_size=ex["block_size"], max_blocks_per_seq=8)
    slots, tables, ctx, cu = pool.step([0], [ex["tokens"]])
    assert len(tables[0]) == ex["blocks"]
    wasted = len(tables[0]) * ex["block_size"] - ex["tokens"]
    assert 0 <= wasted < ex["max_wasted_blocks"] * ex["block_size"]
    assert ctx == [68] and cu == [0, 68] and len(slots) == 68


def check_invariants(pool: BlockPool, num_blocks: int):
    held = [b for t in pool.tables.values() for b in t]
    assert sorted(held + pool.free) == list(range(num_blocks))          # each block once
    seen = {}
    for s, t in pool.tables.items():
        n = pool.lens.get(s, 0)
        assert len(t) == math.ceil(n / pool.block_size)
        for p in range(n):
            slot = pool.slot(s, p)
            assert slot // pool.block_size == t[p // pool.block_size]
            assert slot % pool.block_size == p % pool.block_size
            assert slot not in seen, "two live positions share a slot"
            seen[slot] = (s, p)


@pytest.mark.parametrize("seed", range(6))
def test_random_steps_keep_the_invariants(seed):
    rng = np.random.default_rng(seed)
    nb, bs, W, S = 40, int(rng.choice([1, 3, 4, 16])), 12, 10
    pool = BlockPool(nb, bs, W)
    for _ in range(120):
        if rng.random() < 0.2 and pool.tables:
            pool.release(int(rng.choice(list(pool.tables))))
        else:
            k = int(rng.integers(1, 5))
            seqs = rng.choice(S, size=k, replace=False).tolist()
            num = rng.integers(0, 2 * bs + 2, size=k).tolist()
            before = (list(pool.free), {s: list(t) for s, t in pool.tables.items()}, dict(pool.lens))
            try:
                slots, tables, ctx, cu = pool.step(seqs, num)
            except (NoSpace, ValueError):
                assert (pool.free, pool.tables, pool.lens) == before      # nothing changed
                continue
            assert cu[-1] == len(slots) == sum(num) and len(set(slots)) == len(slots)
            for i, s in enumerate(seqs):                                   # new slots = the chunk's positions
                old = ctx[i] - num[i]
                assert slots[cu[i]:cu[i + 1]] == [pool.slot(s, p) for p in range(old, ctx[i])]
        check_invariants(pool, nb)


def test_out_of_space_changes_nothing():
    pool = BlockPool(5, 4, 8)
    pool.step([0, 1], [9, 4])                 # 3 + 1 blocks
    before = (list(pool.free), {s: list(t) for s, t in pool.tables.items()}, dict(pool.lens))
    with pytest.raises(NoSpace):
        pool.step([1, 2], [1, 4])             # needs 1 + 1, only 1 free
    assert (pool.free, pool.tables, pool.lens) == before


def test_hand_out_order_hand_worked():
    pool = BlockPool(6, 2, 4)
    _, tables, _, _ = pool.step([0, 1], [3, 1])
    assert tables == [[0, 1], [2]]
    pool.release(0)
    assert pool.free == [0, 1, 3, 4, 5]
    slots, tables, ctx, cu = pool.step([2, 1], [5, 2])
    assert tables == [[0, 1, 3], [2, 4]]
    assert slots == [0, 1, 2, 3, 6, 5, 8]     # seq 2 positions 0..4, then seq 1 positions 1, 2
    assert ctx == [5, 3] and cu == [0, 5, 7]


def test_paged_through_the_pool_equals_dense_attention():
    """Chunks written through the pool's slots (oracle write) and read back
    through its tables (oracle prefill attention) give torch SDPA on the
    sequences' dense K/V in position order."""
    rng = np.random.default_rng(11)
    nb, bs, hq, hkv, d = 30, 4, 4, 2, 16
    pool = BlockPool(nb, bs, 10)
    kc = np.zeros((nb, bs, hkv, d), dtype=np.uint16)
    vc = np.zeros_like(kc)
    dense_k = {s: [] for s in range(3)}
    dense_v = {s: [] for s in range(3)}
    for seqs, num in (([0, 1], [6, 3]), ([2, 0], [9, 1]), ([1, 2, 0], [5, 1, 2])):
        sm, bt, cl, cu = pool.step_arrays(seqs, num, 10)
        T = int(cu[-1])
        nk = workloads.normal_bf16_bits(rng, (T, hkv, d))
        nv = workloads.normal_bf16_bits(rng, (T, hkv, d))
        oracle.reshape_and_cache(nk, nv, oracle.BF16, kc, vc, oracle.BF16, sm, None)
        for i, s in enumerate(seqs):
            dense_k[s].extend(nk[cu[i]:cu[i + 1]])
            dense_v[s].extend(nv[cu[i]:cu[i + 1]])
        q = workloads.normal_bf16_bits(rng, (T, hq, d))
        got = oracle.prefill_attention(q, oracle.BF16, cu, kc, vc, oracle.BF16, bt, cl, 0.25)
        f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
        for i, s in enumerate(seqs):
            L, n = int(cl[i]), int(num[i])
            K = torch.from_numpy(f(np.array(dense_k[s]))).permute(1, 0, 2).repeat_interleave(2, 0)
            V = torch.from_numpy(f(np.array(dense_v[s]))).permute(1, 0, 2).repeat_interleave(2, 0)
            qs = torch.from_numpy(f(q[cu[i]:cu[i + 1]])).permute(1, 0, 2)
            pos = L - n + np.arange(n)
            mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
            ref = torch.nn.functional.scaled_dot_product_attention(
                qs.contiguous(), K.contiguous(), V.contiguous(), attn_mask=mask, scale=0.25)
            np.testing.assert_allclose(got[cu[i]:cu[i + 1]], ref.permute(1, 0, 2).numpy(),
                                       rtol=1e-12, atol=1e-12)
