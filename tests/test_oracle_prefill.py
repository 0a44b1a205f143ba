"""Pins of the oracle's fp64 chunked-prefill paged attention (reading R10). CPU only.

Pins: library special cases (torch scaled_dot_product_attention in fp64: with
is_causal for a whole-prompt prefill, with an explicit position mask for a
chunk on top of a cached prefix), the decode oracle for one-token chunks,
closed forms (the first prompt token attends only to itself), paged == dense,
invariance under a permutation of the physical block ids, chunks longer than
the context (leading queries have no key), and the fp8 dequantisation."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def make_prefill(rng, ctx, nq, hq=4, hkv=2, d=16, bs=4, spare=3):
    """Paged caches holding ``ctx[b]`` positions per sequence and ``nq[b]`` packed
    queries per sequence."""
    ctx = np.asarray(ctx, dtype=np.int32)
    nq = np.asarray(nq, dtype=np.int32)
    nblk = [-(-int(c) // bs) for c in ctx]
    nb = sum(nblk) + spare
    W = max(max(nblk), 1) + 1
    perm = rng.permutation(nb).astype(np.int32)
    bt = workloads.deal_block_tables(perm, ctx, bs, W)
    kc = workloads.normal_bf16_bits(rng, (nb, bs, hkv, d))
    vc = workloads.normal_bf16_bits(rng, (nb, bs, hkv, d))
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = workloads.normal_bf16_bits(rng, (int(cu[-1]), hq, d))
    return dict(ctx=ctx, nq=nq, cu=cu, bt=bt, kc=kc, vc=vc, q=q, bs=bs, hq=hq, hkv=hkv, d=d)


def dense(cache_f64, bt, n, bs):
    """K or V of one sequence as [n, H_KV, D]: position p is row p % bs of block bt[p // bs]."""
    pos = np.arange(n)
    return cache_f64[bt[pos // bs], pos % bs]


def sdpa_reference(p, scale, k_mul=1.0, v_mul=1.0, decode=bits_to_f64):
    """torch SDPA per sequence with the chunk's causal mask over the whole context."""
    G = p["hq"] // p["hkv"]
    out = np.zeros(p["q"].shape, dtype=np.float64)
    for b, (L, n) in enumerate(zip(p["ctx"], p["nq"])):
        L, n, t0 = int(L), int(n), int(p["cu"][b])
        if n == 0:
            continue
        K = dense(decode(p["kc"]), p["bt"][b], L, p["bs"]) * k_mul
        V = dense(decode(p["vc"]), p["bt"][b], L, p["bs"]) * v_mul
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        qt = torch.from_numpy(bits_to_f64(p["q"][t0:t0 + n])).permute(1, 0, 2).contiguous()
        pos = L - n + np.arange(n)                       # query positions
        mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask,
                                                             scale=scale)
        out[t0:t0 + n] = o.permute(1, 0, 2).numpy()
    return out


def run_oracle(p, scale, cache_dtype=oracle.BF16, k_scale=None, v_scale=None):
    return oracle.prefill_attention(p["q"], oracle.BF16, p["cu"], p["kc"], p["vc"], cache_dtype,
                                    p["bt"], p["ctx"], scale, k_scale, v_scale)


def test_whole_prompt_is_causal_sdpa():
    """No cached prefix (n_b == ctx_b): torch's is_causal path, independently of the mask builder."""
    rng = np.random.default_rng(3)
    p = make_prefill(rng, [7, 16, 1], [7, 16, 1], hq=4, hkv=2, d=16, bs=4)
    got = run_oracle(p, 0.25)
    G = 2
    for b in range(3):
        L, t0 = int(p["ctx"][b]), int(p["cu"][b])
        K = dense(bits_to_f64(p["kc"]), p["bt"][b], L, 4)
        V = dense(bits_to_f64(p["vc"]), p["bt"][b], L, 4)
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        qt = torch.from_numpy(bits_to_f64(p["q"][t0:t0 + L])).permute(1, 0, 2).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, is_causal=True,
                                                               scale=0.25)
        np.testing.assert_allclose(got[t0:t0 + L], ref.permute(1, 0, 2).numpy(), rtol=1e-12,
                                   atol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 1), (3, 3), (16, 8), (8, 2)])
def test_chunks_on_cached_prefix_match_masked_sdpa(hq, hkv):
    rng = np.random.default_rng(hq * 7 + hkv)
    p = make_prefill(rng, [1, 9, 30, 17, 40], [1, 4, 13, 17, 2], hq=hq, hkv=hkv, d=16, bs=4)
    scale = 1 / math.sqrt(16)
    np.testing.assert_allclose(run_oracle(p, scale), sdpa_reference(p, scale), rtol=1e-12,
                               atol=1e-12)


def test_one_token_chunks_equal_the_decode_oracle():
    rng = np.random.default_rng(5)
    p = make_prefill(rng, [3, 19, 33, 64], [1, 1, 1, 1], hq=8, hkv=4, d=32, bs=8)
    dec = oracle.decode_attention(p["q"], oracle.BF16, p["kc"], p["vc"], oracle.BF16, p["bt"],
                                  p["ctx"], 0.2)
    assert np.array_equal(run_oracle(p, 0.2), dec)


def test_first_prompt_token_reads_its_own_value_row():
    """Position 0 has one key: the softmax weight is 1, the output is V[0] exactly."""
    rng = np.random.default_rng(6)
    p = make_prefill(rng, [5, 12], [5, 12], hq=4, hkv=2, d=8, bs=4)
    got = run_oracle(p, 0.7)
    V = bits_to_f64(p["vc"])
    for b in range(2):
        t0 = int(p["cu"][b])
        v0 = V[p["bt"][b][0], 0]                         # [H_KV, D]
        assert np.array_equal(got[t0], np.repeat(v0, 2, axis=0))


def test_paged_equals_dense_and_relabelling_is_exact():
    rng = np.random.default_rng(8)
    p = make_prefill(rng, [13, 26, 7], [5, 26, 3], hq=4, hkv=2, d=16, bs=4, spare=6)
    base = run_oracle(p, 0.3)
    perm = rng.permutation(p["kc"].shape[0])
    q = dict(p)
    q["kc"] = np.empty_like(p["kc"])
    q["vc"] = np.empty_like(p["vc"])
    q["kc"][perm], q["vc"][perm] = p["kc"], p["vc"]
    q["bt"] = np.where(p["bt"] >= 0, perm[np.maximum(p["bt"], 0)], -1).astype(np.int32)
    assert np.array_equal(run_oracle(q, 0.3), base)
    # dense contiguous layout: one block per sequence holding all its positions in order
    for b in range(3):
        L, t0, n = int(p["ctx"][b]), int(p["cu"][b]), int(p["nq"][b])
        kd = dense(p["kc"], p["bt"][b], L, 4)[None]     # [1, L, H_KV, D] as a single block
        vd = dense(p["vc"], p["bt"][b], L, 4)[None]
        single = oracle.prefill_attention(p["q"][t0:t0 + n], oracle.BF16,
                                          np.array([0, n], dtype=np.int32), kd, vd, oracle.BF16,
                                          np.zeros((1, 1), dtype=np.int32),
                                          np.array([L], dtype=np.int32), 0.3)
        assert np.array_equal(single, base[t0:t0 + n])


def test_chunk_longer_than_context_and_empty_sequences():
    """n_b > ctx_b: the first n_b - ctx_b queries have no key (zeros); empty
    sequences contribute no rows."""
    rng = np.random.default_rng(9)
    p = make_prefill(rng, [3, 8, 0], [5, 0, 2], hq=4, hkv=2, d=8, bs=4)
    got = run_oracle(p, 0.5)
    assert np.all(got[0:2] == 0) and np.all(got[5:7] == 0)
    # rows 2..4 are positions 0..2 of sequence 0
    np.testing.assert_allclose(got[2:5], _tail_reference(p, 0.5), rtol=1e-12, atol=1e-12)


def _tail_reference(p, scale):
    """Sequence 0's last three queries (positions 0..2) as a whole-prompt causal SDPA."""
    K = dense(bits_to_f64(p["kc"]), p["bt"][0], 3, 4)
    V = dense(bits_to_f64(p["vc"]), p["bt"][0], 3, 4)
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(2, dim=0).contiguous()
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(2, dim=0).contiguous()
    qt = torch.from_numpy(bits_to_f64(p["q"][2:5])).permute(1, 0, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, is_causal=True, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_fp8_dequantisation_multiplies_by_the_scales():
    rng = np.random.default_rng(10)
    p = make_prefill(rng, [11, 20], [4, 20], hq=4, hkv=2, d=16, bs=4)
    kc = workloads.normal_fp8_codes(rng, p["kc"].shape, 0.05)
    vc = workloads.normal_fp8_codes(rng, p["vc"].shape, 0.04)
    f8 = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    p8 = dict(p, kc=kc, vc=vc)
    got = run_oracle(p8, 0.25, oracle.FP8_E4M3FN, 0.05, 0.04)
    ref = sdpa_reference(p8, 0.25, k_mul=float(np.float32(0.05)), v_mul=float(np.float32(0.04)),
                         decode=lambda c: f8[c])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
