"""GPU parity of paged decode attention against the fp64 oracle
(|gpu - oracle| <= 2e-3 + 2e-3*|oracle|, GPU output in bf16 unless stated):
small ragged cases over every supported group size, head size and cache type,
the degenerate lengths, bit-identical output under relabelled physical blocks,
and the full Qwen3-0.6B-shaped decode steps (batch 64 bf16 with the new-token
write, batch 256 fp8)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import assert_attention_close, say, sentinel, to_dev, to_host, widen_out

pytestmark = pytest.mark.gpu

BF16, F32, FP8 = oracle.BF16, oracle.F32, oracle.FP8_E4M3FN


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def pkv():
    import paged_kv_cache_304_amd as m
    return m


def gpu_attention(q_bits, kc, vc, cache_dt, bt, ctx, scale, ks=None, vs=None, out_dt=BF16):
    m = pkv()
    q = to_dev(q_bits, BF16)
    out = torch.empty(q.shape, dtype=torch.float32 if out_dt == F32 else torch.bfloat16,
                      device="cuda")
    dk, dv = to_dev(kc, cache_dt), to_dev(vc, cache_dt)
    k_s = None if ks is None else torch.tensor([ks], dtype=torch.float32, device="cuda")
    v_s = None if vs is None else torch.tensor([vs], dtype=torch.float32, device="cuda")
    m.decode_attention(out, q, dk, dv, torch.from_numpy(bt).cuda(), torch.from_numpy(ctx).cuda(),
                       scale, k_s, v_s)
    torch.cuda.synchronize()
    return out


def make_case(seed, ctx, hq, hkv, d, bs, cache_dt, spare=5, width=None):
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    nblk = [-(-int(c) // bs) for c in ctx]
    nb = sum(nblk) + spare
    W = width or max(max(nblk), 1)
    perm = rng.permutation(nb).astype(np.int32)
    bt = workloads.deal_block_tables(perm, ctx, bs, W)
    if cache_dt == FP8:
        kc = workloads.normal_fp8_codes(rng, (nb, bs, hkv, d), 0.05)
        vc = workloads.normal_fp8_codes(rng, (nb, bs, hkv, d), 0.04)
    else:
        kc = workloads.normal_bf16_bits(rng, (nb, bs, hkv, d))
        vc = workloads.normal_bf16_bits(rng, (nb, bs, hkv, d))
    q = workloads.normal_bf16_bits(rng, (len(ctx), hq, d))
    return q, kc, vc, bt, ctx


CASES = [
    # name, ctx list, hq, hkv, d, bs, cache, width
    ("G2 D128 bf16 ragged", [1, 15, 16, 17, 100, 333, 1024, 700], 16, 8, 128, 16, BF16, 80),
    ("G2 D128 fp8 ragged", [1, 16, 63, 257, 999, 2000], 16, 8, 128, 16, FP8, 130),
    ("G1 D128 bf16", [5, 77, 512], 8, 8, 128, 16, BF16, 40),
    ("G4 D128 bf16", [31, 200, 900], 16, 4, 128, 16, BF16, 60),
    ("G8 D128 bf16", [3, 65, 1500], 16, 2, 128, 16, BF16, 100),
    ("G8 D64 fp8", [9, 300, 800], 8, 1, 64, 16, FP8, 60),
    ("G2 D64 bf16 bs8", [1, 8, 9, 411], 4, 2, 64, 8, BF16, 60),
    ("G2 D256 bf16", [2, 33, 600], 8, 4, 256, 16, BF16, 40),
    ("G4 D256 fp8 bs32", [40, 129, 1000], 8, 2, 256, 32, FP8, 40),
    ("G1 D128 bf16 16 kv heads", [70, 3], 16, 16, 128, 16, BF16, 8),
    ("G1 D128 bf16 12 kv heads (idle waves)", [300, 40, 129], 12, 12, 128, 16, BF16, 20),
    # fp8 caches run four KV heads per workgroup, bf16 two: head counts that leave
    # idle waves in the last workgroup, or a workgroup of three waves
    ("G2 D128 fp8 6 kv heads (idle waves)", [300, 40, 129, 1], 12, 6, 128, 16, FP8, 20),
    ("G2 D128 fp8 3 kv heads (3-wave workgroup)", [500, 17, 64], 6, 3, 128, 16, FP8, 32),
    ("G1 D64 fp8 5 kv heads", [222, 1000, 2], 5, 5, 64, 16, FP8, 64),
    ("G1 D64 bf16 3 kv heads (idle wave)", [150, 31, 600], 3, 3, 64, 16, BF16, 40),
    # one GPU's share of the batch-64 workload under 2-way tensor parallelism
    ("G2 D128 bf16 tp2 shard", [1469, 1841, 856, 3464, 17], 8, 4, 128, 16, BF16, 224),
    ("G2 D128 fp8 bs32", [31, 32, 33, 700], 16, 8, 128, 32, FP8, 24),
    ("G2 D128 bf16 one seq long", [4096], 16, 8, 128, 16, BF16, 256),
    ("G2 D128 bf16 many short", list(range(1, 65)), 16, 8, 128, 16, BF16, 4),
    ("G2 D128 bf16 bs64", [1, 63, 64, 65, 3000], 16, 8, 128, 64, BF16, 48),
    ("G4 D64 fp8 bs128", [129, 5, 2100], 8, 2, 64, 128, FP8, 20),
    # 300 sequences (several per scan thread), every third one empty, lengths
    # that cut the tile ranges at many different offsets
    ("G2 D128 bf16 300 seqs with empties", [0 if i % 3 == 0 else 1 + (i * 37) % 700 for i in range(300)],
     16, 8, 128, 16, BF16, 44),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_matches_oracle(case):
    name, ctx, hq, hkv, d, bs, cache_dt, width = case
    say(f"decode_attention {name} B={len(ctx)} H_Q={hq} H_KV={hkv} D={d} bs={bs}")
    q, kc, vc, bt, ctx = make_case(zlib.crc32(name.encode()), ctx, hq, hkv, d, bs, cache_dt,
                                   width=width)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ks, vs = (0.05, 0.04) if cache_dt == FP8 else (None, None)
    ref = oracle.decode_attention(q, BF16, kc, vc, cache_dt, bt, ctx, scale, ks, vs)
    for out_dt in (F32, BF16):
        got = widen_out(gpu_attention(q, kc, vc, cache_dt, bt, ctx, scale, ks, vs, out_dt))
        assert_attention_close(got, ref, f"{name} out={'f32' if out_dt == F32 else 'bf16'}",
                               out_bf16=out_dt == BF16)


def test_degenerate_lengths_and_bad_table_entries():
    """ctx 0 (zeros), ctx beyond the table (clamped), a table entry outside the pool
    (its positions drop out), a length that fills the table exactly."""
    say("decode_attention degenerate lengths")
    q, kc, vc, bt, ctx = make_case(9, [0, 20, 64, 50, 33], 8, 4, 128, 16, BF16, width=4)
    ctx = np.array([0, 20, 64, 5000, 33], dtype=np.int32)   # 5000 > W*bs = 64
    bt = bt.copy()
    bt[4, 1] = kc.shape[0] + 7                              # outside the pool
    bt[1, 1] = -3
    ref = oracle.decode_attention(q, BF16, kc, vc, BF16, bt, ctx, 0.1)
    got = widen_out(gpu_attention(q, kc, vc, BF16, bt, ctx, 0.1))
    assert np.all(got[0] == 0)
    assert_attention_close(got, ref, "degenerate")


def test_unwritten_slots_hold_nan_and_are_masked():
    """The tiny two-sequence workload written by the GPU into NaN-filled caches, then
    attended: the last partial blocks hold NaN outside the context and must not leak."""
    say("decode_attention tiny workload after GPU write into NaN caches")
    m = pkv()
    w = workloads.tiny_paged()
    shape = (w["num_blocks"], w["block_size"], w["num_kv_heads"], w["head_size"])
    okc = np.full(shape, 0x7FC0, dtype=np.uint16)
    ovc = np.full(shape, 0x7FC0, dtype=np.uint16)
    oracle.reshape_and_cache(w["key"], w["value"], BF16, okc, ovc, BF16, w["slot_mapping"])
    ref = oracle.decode_attention(w["q"], BF16, okc, ovc, BF16, w["block_tables"],
                                  w["context_lens"], w["softmax_scale"])
    gk = to_dev(np.full(shape, 0x7FC0, dtype=np.uint16), BF16)
    gv = to_dev(np.full(shape, 0x7FC0, dtype=np.uint16), BF16)
    m.reshape_and_cache(to_dev(w["key"], BF16), to_dev(w["value"], BF16), gk, gv,
                        torch.from_numpy(w["slot_mapping"]).cuda())
    out = torch.empty((2, 16, 128), dtype=torch.bfloat16, device="cuda")
    m.decode_attention(out, to_dev(w["q"], BF16), gk, gv, torch.from_numpy(w["block_tables"]).cuda(),
                       torch.from_numpy(w["context_lens"]).cuda(), w["softmax_scale"])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(gk, BF16), okc)
    assert_attention_close(widen_out(out), ref, "tiny")


@pytest.mark.parametrize("cache_dt", [BF16, FP8])
def test_block_relabelling_is_bit_identical(cache_dt):
    say(f"decode_attention block relabelling cache={'fp8' if cache_dt == FP8 else 'bf16'}")
    q, kc, vc, bt, ctx = make_case(21, [5, 300, 1234, 64], 16, 8, 128, 16, cache_dt, spare=20,
                                   width=80)
    ks, vs = (0.05, 0.04) if cache_dt == FP8 else (None, None)
    a = gpu_attention(q, kc, vc, cache_dt, bt, ctx, 0.088, ks, vs)
    perm = np.random.default_rng(1).permutation(kc.shape[0])
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    b = gpu_attention(q, kc2, vc2, cache_dt, bt2, ctx, 0.088, ks, vs)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_repeated_calls_reuse_workspace():
    """Calls in a row with one workspace (later ones with fewer sequences) match the
    oracle: the workspace carries nothing between calls."""
    say("decode_attention workspace reuse")
    m = pkv()
    q, kc, vc, bt, ctx = make_case(33, [900, 17, 2500, 64, 1], 16, 8, 128, 16, BF16, width=160)
    need = m.decode_attention_workspace_size(5, 16, 8, 128, 160, 16)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # garbage on entry
    dk, dv = to_dev(kc, BF16), to_dev(vc, BF16)
    for n in (5, 3, 5, 1, 5):
        qq = to_dev(q[:n], BF16)
        out = torch.empty_like(qq)
        m.decode_attention(out, qq, dk, dv, torch.from_numpy(bt[:n].copy()).cuda(),
                           torch.from_numpy(ctx[:n].copy()).cuda(), 0.088, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.decode_attention(q[:n], BF16, kc, vc, BF16, bt[:n], ctx[:n], 0.088)
        assert_attention_close(widen_out(out), ref, f"reuse n={n}")


def _full_decode(w: workloads.DecodeWorkload, with_write: bool):
    """Build the workload's pool on the GPU, optionally write the new tokens, run
    attention; return everything the oracle needs on the host."""
    m = pkv()
    B, HQ, HKV, D, BS, NB = (w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size,
                             w.block_size, w.num_blocks)
    if w.cache_dtype == "fp8":
        kc = workloads.device_fp8((NB, BS, HKV, D), "cuda", w.seed, w.k_scale)
        vc = workloads.device_fp8((NB, BS, HKV, D), "cuda", w.seed + 1, w.v_scale)
        cdt = FP8
    else:
        kc = workloads.device_normal((NB, BS, HKV, D), torch.bfloat16, "cuda", w.seed)
        vc = workloads.device_normal((NB, BS, HKV, D), torch.bfloat16, "cuda", w.seed + 1)
        cdt = BF16
    q = workloads.device_normal((B, HQ, D), torch.bfloat16, "cuda", w.seed + 2)
    kc_host = to_host(kc, cdt)
    vc_host = to_host(vc, cdt)
    new_k = new_v = None
    if with_write:
        new_k = workloads.device_normal((B, HKV, D), torch.bfloat16, "cuda", w.seed + 3)
        new_v = workloads.device_normal((B, HKV, D), torch.bfloat16, "cuda", w.seed + 4)
        m.reshape_and_cache(new_k, new_v, kc, vc, torch.from_numpy(w.new_token_slots).cuda())
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.context_lens).cuda()
    ks = None if w.k_scale is None else torch.tensor([w.k_scale], dtype=torch.float32, device="cuda")
    vs = None if w.v_scale is None else torch.tensor([w.v_scale], dtype=torch.float32, device="cuda")
    out = torch.empty((B, HQ, D), dtype=torch.bfloat16, device="cuda")
    m.decode_attention(out, q, kc, vc, bt, cl, w.softmax_scale, ks, vs)
    out32 = torch.empty((B, HQ, D), dtype=torch.float32, device="cuda")
    m.decode_attention(out32, q, kc, vc, bt, cl, w.softmax_scale, ks, vs)
    torch.cuda.synchronize()
    host = dict(out32=widen_out(out32), q=to_host(q, BF16), kc=kc_host, vc=vc_host, cdt=cdt,
                new_k=None if new_k is None else to_host(new_k, BF16),
                new_v=None if new_v is None else to_host(new_v, BF16),
                gpu_kc=to_host(kc, cdt) if with_write else None)
    return out, host


def test_qwen3_decode_b64_full_step():
    """Batch 64, ctx ~ U{512..4096}, 32,768-block bf16 pool: write the 64 new tokens,
    then attend; all 64 x 16 heads are compared with the oracle, with an fp32
    output at the plain bound and with the bf16 output."""
    w = workloads.qwen3_decode_b64()
    say(f"decode step full size {w.name} kv_bytes={w.kv_read_bytes()}")
    out, h = _full_decode(w, with_write=True)
    kc, vc = h["kc"], h["vc"]
    oracle.reshape_and_cache(h["new_k"], h["new_v"], BF16, kc, vc, BF16, w.new_token_slots)
    assert np.array_equal(h["gpu_kc"], kc)  # the GPU write of the step is bit-exact
    ref = oracle.decode_attention(h["q"], BF16, kc, vc, BF16, w.block_tables, w.context_lens,
                                  w.softmax_scale)
    say(f"{w.name}: max |o| {np.abs(ref).max():.3f}, max |err| fp32 out "
        f"{np.abs(h['out32'] - ref).max():.2e}")
    assert_attention_close(h["out32"], ref, w.name + " out=f32", out_bf16=False)
    assert_attention_close(widen_out(out), ref, w.name + " out=bf16")


def test_mixed_decode_fp8_b256_full():
    """Batch 256, lognormal ctx (median 1024, cap 8192), 65,536-block fp8 pool with
    per-tensor scales 0.05/0.04; every output compared with the oracle (fp32 output at
    the plain bound, and the bf16 output)."""
    w = workloads.mixed_decode_fp8()
    say(f"decode full size {w.name} kv_bytes={w.kv_read_bytes()}")
    out, h = _full_decode(w, with_write=False)
    ref = oracle.decode_attention(h["q"], BF16, h["kc"], h["vc"], FP8, w.block_tables,
                                  w.context_lens, w.softmax_scale, w.k_scale, w.v_scale)
    say(f"{w.name}: max |o| {np.abs(ref).max():.3f}, max |err| fp32 out "
        f"{np.abs(h['out32'] - ref).max():.2e}")
    assert_attention_close(h["out32"], ref, w.name + " out=f32", out_bf16=False)
    assert_attention_close(widen_out(out), ref, w.name + " out=bf16")


def test_long_contexts_several_ranges_per_workgroup():
    """40 sequences of 16,384 positions (fp8, 8 KV heads): more tiles per KV-head
    group than 64 per resident workgroup of a 256-CU device, so workgroups take
    several ranges; 8 sampled sequences are compared with the oracle."""
    m = pkv()
    B, HQ, HKV, D, BS, L = 40, 16, 8, 128, 16, 16384
    W = L // BS
    NB = B * W + 16
    say(f"decode_attention long contexts B={B} ctx={L} fp8 pool={NB} blocks")
    rng = workloads.rng_for(40)
    perm = rng.permutation(NB).astype(np.int32)
    ctx = np.full(B, L, dtype=np.int32)
    ctx[7] = L - 5
    bt = workloads.deal_block_tables(perm, ctx, BS, W)
    kc = workloads.device_fp8((NB, BS, HKV, D), "cuda", 4001, 0.05)
    vc = workloads.device_fp8((NB, BS, HKV, D), "cuda", 4002, 0.04)
    q = workloads.device_normal((B, HQ, D), torch.bfloat16, "cuda", 4003)
    ks = torch.tensor([0.05], dtype=torch.float32, device="cuda")
    vs = torch.tensor([0.04], dtype=torch.float32, device="cuda")
    out = torch.empty((B, HQ, D), dtype=torch.float32, device="cuda")
    m.decode_attention(out, q, kc, vc, torch.from_numpy(bt).cuda(), torch.from_numpy(ctx).cuda(),
                       0.088, ks, vs)
    torch.cuda.synchronize()
    sub = np.array([0, 7, 13, 20, 26, 31, 38, 39])
    ref = oracle.decode_attention(to_host(q, BF16)[sub], BF16, to_host(kc, FP8), to_host(vc, FP8), FP8,
                                  bt[sub], ctx[sub], 0.088, 0.05, 0.04)
    assert_attention_close(out.cpu().numpy()[sub].astype(np.float64), ref, "long contexts",
                           out_bf16=False)
