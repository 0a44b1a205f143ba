"""Pins of the oracle's slot resolution, cache write and K concat. CPU only."""
import json
import os

import numpy as np
import torch

import oracle
import workloads

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def test_worked_source_offsets_from_page():
    """Token 5, head 3 of an [T, 8, 128] source starts at element 5504 and ends at 5631."""
    g = GOLDEN["store_kvcache_source_offsets"]
    H, D = g["num_kv_heads"], g["head_dim"]
    T = g["token"] + 2
    key = np.arange(T * H * D, dtype=np.float32).reshape(T, H, D)  # value = flat index
    nb, bs = 4, 16
    kc = np.full((nb, bs, H, D), -1.0, dtype=np.float32)
    slots = np.full(T, -1, dtype=np.int64)
    slots[g["token"]] = 2 * bs + 5  # block 2, offset 5
    n = oracle.reshape_and_cache(key, None, oracle.F32, kc, None, oracle.F32, slots)
    assert n == 1
    got = kc[2, 5, g["head"]]
    assert got[0] == g["first"] and got[-1] == g["last"]
    assert g["token_part"] == g["token"] * H * D and g["head_part"] == g["head"] * D
    assert np.array_equal(got, np.arange(g["first"], g["last"] + 1, dtype=np.float32))
    # the flat cache offset of the page's formula: blk*bs*H*D + off*H*D + h*D + d
    flat = np.flatnonzero(kc.ravel() >= 0)
    assert flat[0] == 2 * bs * H * D + 5 * H * D + 0 and flat.size == H * D


def test_block_allocation_example_from_page():
    """68 tokens at block_size 32 land in exactly 3 blocks, at most one partly used."""
    g = GOLDEN["block_allocation"]
    bs, T = g["block_size"], g["tokens"]
    rng = np.random.default_rng(0)
    perm = rng.permutation(10).astype(np.int32)
    bt = workloads.deal_block_tables(perm, np.array([T], dtype=np.int32), bs, 4)
    slots = workloads.slots_for_positions(bt, np.zeros(T, dtype=np.int64), np.arange(T), bs)
    final = oracle.resolve_slots(slots, 10, bs)
    blocks = np.unique(final // bs)
    assert blocks.size == g["blocks"]
    fill = [np.sum(final // bs == b) for b in blocks]
    assert sum(f < bs for f in fill) <= g["max_wasted_blocks"]


def test_resolve_slots_rules():
    sm = np.array([5, -1, 3, 40, 7, -7, 0], dtype=np.int64)
    # no SWA: negatives and slots beyond the pool (4 blocks of 8) are skipped
    assert list(oracle.resolve_slots(sm, 4, 8)) == [5, -1, 3, -1, 7, -1, 0]
    # with SWA: first-stage negative skips before the table; index >= len skips
    swa = np.array([9, 2, 1, -1, 4, 31, 6, 32], dtype=np.int64)
    assert list(oracle.resolve_slots(sm, 4, 8, swa)) == [31, -1, -1, -1, -1, -1, 9]


def _sentinel_cache(shape, dtype, byte):
    c = np.empty(shape, dtype=dtype)
    c.view(np.uint8)[...] = byte
    return c


def test_round_trip_gather_returns_written_bits():
    """Write the tiny two-sequence workload, then gather every (sequence, position)
    back through the block table: the bits come back unchanged, and every slot that
    was not written still holds the sentinel."""
    w = workloads.tiny_paged()
    shape = (w["num_blocks"], w["block_size"], w["num_kv_heads"], w["head_size"])
    kc = _sentinel_cache(shape, np.uint16, 0xA5)
    vc = _sentinel_cache(shape, np.uint16, 0xA5)
    n = oracle.reshape_and_cache(w["key"], w["value"], oracle.BF16, kc, vc, oracle.BF16,
                                 w["slot_mapping"])
    assert n == w["slot_mapping"].shape[0]
    bt, bs = w["block_tables"], w["block_size"]
    t = 0
    written = np.zeros(shape[:2], dtype=bool)
    for b, ctx in enumerate(w["context_lens"]):
        for p in range(ctx):
            blk, off = bt[b, p // bs], p % bs
            assert np.array_equal(kc[blk, off], w["key"][t])
            assert np.array_equal(vc[blk, off], w["value"][t])
            written[blk, off] = True
            t += 1
    assert np.all(kc[~written].view(np.uint8) == 0xA5) and np.all(vc[~written].view(np.uint8) == 0xA5)


def test_fp8_write_matches_library_per_element_and_skips():
    rng = np.random.default_rng(3)
    T, H, D, nb, bs = 50, 2, 16, 8, 8
    key = workloads.normal_bf16_bits(rng, (T, H, D), std=2.0)
    val = workloads.normal_bf16_bits(rng, (T, H, D), std=2.0)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[[3, 17, 40]] = -1
    kc = _sentinel_cache((nb, bs, H, D), np.uint8, 0x7F)
    vc = _sentinel_cache((nb, bs, H, D), np.uint8, 0x7F)
    oracle.reshape_and_cache(key, val, oracle.BF16, kc, vc, oracle.FP8_E4M3FN, slots,
                             k_scale=0.05, v_scale=0.04)
    kf = torch.from_numpy((key.astype(np.uint32) << 16).view(np.float32).copy())
    vf = torch.from_numpy((val.astype(np.uint32) << 16).view(np.float32).copy())
    kref = (kf / torch.tensor(0.05)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    vref = (vf / torch.tensor(0.04)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for t in range(T):
        if slots[t] < 0:
            continue
        blk, off = divmod(int(slots[t]), bs)
        assert np.array_equal(kc[blk, off], kref[t]) and np.array_equal(vc[blk, off], vref[t])
    untouched = np.ones(nb * bs, dtype=bool)
    untouched[slots[slots >= 0]] = False
    assert np.all(kc.reshape(nb * bs, -1)[untouched] == 0x7F)


def test_swa_write_and_token_stride():
    """Second-stage table and a padded source row (token stride > H*D)."""
    rng = np.random.default_rng(4)
    T, H, D, nb, bs = 24, 3, 8, 4, 8
    src = np.arange(T * (H * D + 5), dtype=np.float32).reshape(T, H * D + 5)
    slots = rng.permutation(T).astype(np.int64)
    swa = rng.permutation(nb * bs)[:T].astype(np.int64)
    swa[[1, 5]] = -1
    kc = np.full((nb, bs, H, D), -1.0, dtype=np.float32)
    oracle.reshape_and_cache(src, None, oracle.F32, kc, None, oracle.F32,
                             slots, swa_slot_mapping=swa, key_token_stride=H * D + 5)
    for t in range(T):
        fin = swa[slots[t]]
        if fin < 0:
            continue
        blk, off = divmod(int(fin), bs)
        assert np.array_equal(kc[blk, off].ravel(), src[t, :H * D])


def test_f32_to_bf16_write_matches_torch():
    rng = np.random.default_rng(8)
    T, H, D, nb, bs = 20, 2, 8, 4, 8
    x = (rng.standard_normal((T, H, D)) * 3).astype(np.float32)
    kc = np.zeros((nb, bs, H, D), dtype=np.uint16)
    slots = np.arange(T, dtype=np.int64)
    oracle.reshape_and_cache(x, None, oracle.F32, kc, None, oracle.BF16, slots)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kc.reshape(-1, H, D)[:T], ref)


def test_concat_closed_form_and_round_trip():
    """bf16 -> fp32 widening is a 16-bit shift of the pattern; rope is shared by all
    heads; casting the fp32 result back to bf16 returns the inputs' bits."""
    rng = np.random.default_rng(9)
    T, H, nope, rope = 7, 5, 16, 8
    kn = workloads.normal_bf16_bits(rng, (T, H, nope))
    kr = workloads.normal_bf16_bits(rng, (T, 1, rope))
    k = np.zeros((T, H, nope + rope), dtype=np.float32)
    oracle.concat_and_cast(k, oracle.F32, kn, oracle.BF16, kr, oracle.BF16)
    bits = k.view(np.uint32)
    assert np.array_equal(bits[:, :, :nope], kn.astype(np.uint32) << 16)
    assert np.array_equal(bits[:, :, nope:], np.broadcast_to(kr.astype(np.uint32) << 16,
                                                            (T, H, rope)))
    # bf16 -> bf16 is a copy, into a strided destination
    k2 = np.zeros((T, H + 1, nope + rope + 3), dtype=np.uint16)[:, :H, :nope + rope]
    oracle.concat_and_cast(k2, oracle.BF16, kn, oracle.BF16, kr, oracle.BF16)
    assert np.array_equal(k2[:, :, :nope], kn)
    assert np.array_equal(k2[:, :, nope:], np.broadcast_to(kr, (T, H, rope)))
    # round trip through the K-only bf16 write
    kc = np.zeros((2, 8, H, nope + rope), dtype=np.uint16)
    oracle.reshape_and_cache(k, None, oracle.F32, kc, None, oracle.BF16,
                             np.arange(T, dtype=np.int64))
    assert np.array_equal(kc.reshape(-1, H, nope + rope)[:T], k2)
