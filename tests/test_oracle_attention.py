"""Pins of the oracle's fp64 paged decode attention. CPU only.

Pins: a library special case (torch scaled_dot_product_attention in fp64 over
the gathered, head-repeated K/V), closed forms (one position, identical keys,
one dominant logit), paged == dense, invariance under a permutation of the
physical block ids, the empty sequence, and the fp8 dequantisation."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def make_paged(rng, ctx, hq=4, hkv=2, d=16, bs=4, nb=None, spare=3):
    ctx = np.asarray(ctx, dtype=np.int32)
    nblk = [-(-int(c) // bs) for c in ctx]
    nb = nb or (sum(nblk) + spare)
    W = max(max(nblk), 1) + 1
    perm = rng.permutation(nb).astype(np.int32)
    bt = workloads.deal_block_tables(perm, ctx, bs, W)
    kc = workloads.normal_bf16_bits(rng, (nb, bs, hkv, d))
    vc = workloads.normal_bf16_bits(rng, (nb, bs, hkv, d))
    q = workloads.normal_bf16_bits(rng, (len(ctx), hq, d))
    return dict(ctx=ctx, bt=bt, kc=kc, vc=vc, q=q, bs=bs, hq=hq, hkv=hkv, d=d, nb=nb)


def gather_dense(cache_f64, bt, ctx, bs):
    """K or V of one sequence as [ctx, H_KV, D] through its block table."""
    pos = np.arange(ctx)
    return cache_f64[bt[pos // bs], pos % bs]


def sdpa_reference(p, scale, k_mul=1.0, v_mul=1.0, decode=bits_to_f64):
    out = []
    G = p["hq"] // p["hkv"]
    for b, c in enumerate(p["ctx"]):
        K = gather_dense(decode(p["kc"]), p["bt"][b], int(c), p["bs"]) * k_mul
        V = gather_dense(decode(p["vc"]), p["bt"][b], int(c), p["bs"]) * v_mul
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [HQ, ctx, D]
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qt = torch.from_numpy(bits_to_f64(p["q"][b]))[:, None, :]              # [HQ, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(qt, Kt.contiguous(), Vt.contiguous(),
                                                             scale=scale)
        out.append(o[:, 0, :].numpy())
    return np.stack(out)


def run_oracle(p, scale, cache_dtype=oracle.BF16, k_scale=None, v_scale=None):
    return oracle.decode_attention(p["q"], oracle.BF16, p["kc"], p["vc"], cache_dtype, p["bt"],
                                   p["ctx"], scale, k_scale, v_scale)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 1), (3, 3), (16, 8)])
def test_matches_sdpa_fp64(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    p = make_paged(rng, [1, 5, 17, 32], hq=hq, hkv=hkv, d=16, bs=4)
    scale = 1 / math.sqrt(16)
    got = run_oracle(p, scale)
    ref = sdpa_reference(p, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_group_mapping_is_contiguous_not_interleaved():
    """The SDPA pin separates h // G from h % H_KV: the interleaved mapping differs."""
    rng = np.random.default_rng(1)
    p = make_paged(rng, [9, 12], hq=4, hkv=2, d=8, bs=4)
    got = run_oracle(p, 0.3)
    wrong = dict(p)
    wrong_q = p["q"].copy()
    wrong_q[:, [1, 2]] = p["q"][:, [2, 1]]  # swapping heads 1,2 emulates h % H_KV
    wrong["q"] = wrong_q
    alt = sdpa_reference(wrong, 0.3)[:, [0, 2, 1, 3]]
    assert not np.allclose(got, alt, atol=1e-6)
    np.testing.assert_allclose(got, sdpa_reference(p, 0.3), rtol=1e-12, atol=1e-12)


def test_single_position_returns_that_value_row_exactly():
    rng = np.random.default_rng(2)
    p = make_paged(rng, [1, 1], hq=4, hkv=2, d=16, bs=4)
    got = run_oracle(p, 0.25)
    for b in range(2):
        v = gather_dense(bits_to_f64(p["vc"]), p["bt"][b], 1, 4)[0]  # [HKV, D]
        assert np.array_equal(got[b], np.repeat(v, 2, axis=0))


def test_identical_keys_average_the_values():
    rng = np.random.default_rng(3)
    p = make_paged(rng, [13], hq=2, hkv=1, d=8, bs=4)
    p["kc"][...] = p["kc"][0, 0]  # one key everywhere
    got = run_oracle(p, 0.7)
    V = gather_dense(bits_to_f64(p["vc"]), p["bt"][0], 13, 4)
    np.testing.assert_allclose(got[0], np.repeat(V.mean(axis=0), 2, axis=0), rtol=0, atol=1e-14)


def test_dominant_logit_selects_its_value_row():
    rng = np.random.default_rng(4)
    p = make_paged(rng, [10], hq=1, hkv=1, d=8, bs=4)
    q = bits_to_f64(p["q"][0, 0])
    # position 6 gets the key 64*sign(q); all others get zero keys
    p["kc"][...] = 0
    blk, off = p["bt"][0, 6 // 4], 6 % 4
    p["kc"][blk, off, 0] = workloads.bf16_bits_from_f32(np.sign(q).astype(np.float32) * 64)
    got = run_oracle(p, 1.0)
    V = gather_dense(bits_to_f64(p["vc"]), p["bt"][0], 10, 4)
    np.testing.assert_allclose(got[0, 0], V[6, 0], rtol=0, atol=1e-12)


def test_paged_equals_dense_and_block_permutation_invariance():
    rng = np.random.default_rng(5)
    p = make_paged(rng, [7, 16, 30], hq=4, hkv=2, d=16, bs=4, spare=5)
    got = run_oracle(p, 0.2)
    # dense: the same tokens in consecutive blocks 0.. of a fresh pool
    dense = dict(p)
    nblk = [-(-int(c) // 4) for c in p["ctx"]]
    W = p["bt"].shape[1]
    bt_dense = np.full_like(p["bt"], -1)
    kc_d = np.zeros_like(p["kc"])
    vc_d = np.zeros_like(p["vc"])
    nxt = 0
    for b, n in enumerate(nblk):
        for j in range(n):
            bt_dense[b, j] = nxt
            kc_d[nxt] = p["kc"][p["bt"][b, j]]
            vc_d[nxt] = p["vc"][p["bt"][b, j]]
            nxt += 1
    dense.update(bt=bt_dense, kc=kc_d, vc=vc_d)
    assert np.array_equal(run_oracle(dense, 0.2), got)
    # random relabelling of the physical blocks, data moved with them
    perm = rng.permutation(p["nb"])
    moved = dict(p)
    kc_p = np.empty_like(p["kc"])
    vc_p = np.empty_like(p["vc"])
    kc_p[perm] = p["kc"]
    vc_p[perm] = p["vc"]
    bt_p = np.where(p["bt"] >= 0, perm[np.maximum(p["bt"], 0)], -1).astype(np.int32)
    moved.update(bt=bt_p, kc=kc_p, vc=vc_p)
    assert np.array_equal(run_oracle(moved, 0.2), got)
    assert W == bt_p.shape[1]


def test_empty_sequence_and_invalid_table_entry():
    rng = np.random.default_rng(6)
    p = make_paged(rng, [0, 8], hq=2, hkv=1, d=8, bs=4)
    got = run_oracle(p, 0.5)
    assert np.all(got[0] == 0)
    # an entry outside the pool drops its positions from the softmax
    p2 = dict(p)
    bt = p["bt"].copy()
    bt[1, 1] = p["nb"] + 100
    p2["bt"] = bt
    got2 = run_oracle(p2, 0.5)
    only_first = dict(p)
    only_first["ctx"] = np.array([0, 4], dtype=np.int32)
    np.testing.assert_allclose(got2, run_oracle(only_first, 0.5), rtol=0, atol=0)


def test_fp8_cache_dequantised_by_scales():
    rng = np.random.default_rng(7)
    p = make_paged(rng, [9, 21], hq=4, hkv=2, d=16, bs=4)
    p["kc"] = workloads.normal_fp8_codes(rng, p["kc"].shape, 0.05)
    p["vc"] = workloads.normal_fp8_codes(rng, p["vc"].shape, 0.04)
    ks, vs = float(np.float32(0.05)), float(np.float32(0.04))
    got = run_oracle(p, 0.25, oracle.FP8_E4M3FN, ks, vs)

    def dec(c):
        return torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()

    ref = sdpa_reference(p, 0.25, k_mul=ks, v_mul=vs, decode=dec)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_tiny_workload_written_then_attended_matches_sdpa():
    """The two-sequence workload end to end: oracle write, then oracle attention."""
    w = workloads.tiny_paged()
    shape = (w["num_blocks"], w["block_size"], w["num_kv_heads"], w["head_size"])
    kc = np.full(shape, 0x7FC0, dtype=np.uint16)
    vc = np.full(shape, 0x7FC0, dtype=np.uint16)  # NaN sentinel outside written slots
    oracle.reshape_and_cache(w["key"], w["value"], oracle.BF16, kc, vc, oracle.BF16,
                             w["slot_mapping"])
    p = dict(ctx=w["context_lens"], bt=w["block_tables"], kc=kc, vc=vc, q=w["q"],
             bs=w["block_size"], hq=w["num_q_heads"], hkv=w["num_kv_heads"], d=w["head_size"])
    got = run_oracle(p, w["softmax_scale"])
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, sdpa_reference(p, w["softmax_scale"]), rtol=1e-12, atol=1e-12)
