"""GPU parity of the fused decode step (new-token write + decode attention in
one call) against the oracle's write followed by its attention: the caches
after the step bit-exact, the output within the attention tolerance; the full
batch-64 step bit-identical to the two separate GPU calls; and the step
captured in a HIP graph, replayed with eager work in between, equal to eager
on every replay."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import assert_attention_close, say, to_dev, to_host, widen_out

pytestmark = pytest.mark.gpu

BF16, F32, FP8 = oracle.BF16, oracle.F32, oracle.FP8_E4M3FN
NAN_BF16, NAN_FP8 = 0x7FC0, 0x7F


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def pkv():
    import paged_kv_cache_304_amd as m
    return m


def make_step(seed, ctx, hq, hkv, d, bs, cache_dt, spare=6, slot_mode="table"):
    """Pool holding positions 0..ctx-2 of each sequence; the slot of position
    ctx-1 holds NaN until the step writes it. slot_mode: 'table' (the new token's
    slot is that position's slot), 'skip' (-1: nothing written; the slot then
    holds finite old data), 'elsewhere' (a spare slot no context reads)."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    B = len(ctx)
    nblk = [-(-int(c) // bs) for c in ctx]
    nb = sum(nblk) + spare
    W = max(max(nblk), 1)
    perm = rng.permutation(nb).astype(np.int32)
    bt = workloads.deal_block_tables(perm, ctx, bs, W)
    if cache_dt == FP8:
        kc = workloads.normal_fp8_codes(rng, (nb, bs, hkv, d), 0.05)
        vc = workloads.normal_fp8_codes(rng, (nb, bs, hkv, d), 0.04)
        nan = NAN_FP8
    else:
        kc = workloads.normal_bf16_bits(rng, (nb, bs, hkv, d))
        vc = workloads.normal_bf16_bits(rng, (nb, bs, hkv, d))
        nan = NAN_BF16
    new_slots = np.full(B, -1, dtype=np.int64)
    referenced = set(bt[bt >= 0].tolist())
    free = [s for s in range(nb * bs) if s // bs not in referenced]  # slots no context reads
    used = set()
    for b, c in enumerate(ctx):
        if c == 0:
            new_slots[b] = free.pop()    # an empty sequence still writes its new token
        if c > 0:
            p = int(c) - 1
            s = int(bt[b, p // bs]) * bs + p % bs
            used.add(s)
            if slot_mode != "skip":
                kc.reshape(nb * bs, hkv, d)[s] = nan
                vc.reshape(nb * bs, hkv, d)[s] = nan
            new_slots[b] = s
    if slot_mode == "skip":
        new_slots[::2] = -1
    elif slot_mode == "elsewhere":
        for b in range(0, B, 2):
            new_slots[b] = free.pop()
        for b in range(0, B, 2):   # the attention then reads the old (finite) value at ctx-1
            if ctx[b] > 0:
                p = int(ctx[b]) - 1
                s = int(bt[b, p // bs]) * bs + p % bs
                kc.reshape(nb * bs, hkv, d)[s] = workloads.normal_fp8_codes(rng, (hkv, d), 0.05) \
                    if cache_dt == FP8 else workloads.normal_bf16_bits(rng, (hkv, d))
                vc.reshape(nb * bs, hkv, d)[s] = workloads.normal_fp8_codes(rng, (hkv, d), 0.04) \
                    if cache_dt == FP8 else workloads.normal_bf16_bits(rng, (hkv, d))
    new_k = workloads.normal_bf16_bits(rng, (B, hkv, d))
    new_v = workloads.normal_bf16_bits(rng, (B, hkv, d))
    q = workloads.normal_bf16_bits(rng, (B, hq, d))
    return dict(q=q, kc=kc, vc=vc, bt=bt, ctx=ctx, new_k=new_k, new_v=new_v, new_slots=new_slots)


def gpu_step(c, cache_dt, scale, ks=None, vs=None, out_dt=BF16):
    m = pkv()
    dk, dv = to_dev(c["kc"], cache_dt), to_dev(c["vc"], cache_dt)
    q = to_dev(c["q"], BF16)
    out = torch.empty(q.shape, dtype=torch.float32 if out_dt == F32 else torch.bfloat16, device="cuda")
    k_s = None if ks is None else torch.tensor([ks], dtype=torch.float32, device="cuda")
    v_s = None if vs is None else torch.tensor([vs], dtype=torch.float32, device="cuda")
    m.decode_step(to_dev(c["new_k"], BF16), to_dev(c["new_v"], BF16),
                  torch.from_numpy(c["new_slots"]).cuda(), out, q, dk, dv,
                  torch.from_numpy(c["bt"]).cuda(), torch.from_numpy(c["ctx"]).cuda(), scale, k_s, v_s)
    torch.cuda.synchronize()
    return out, to_host(dk, cache_dt), to_host(dv, cache_dt)


def oracle_step(c, cache_dt, scale, ks=None, vs=None):
    okc, ovc = c["kc"].copy(), c["vc"].copy()
    oracle.reshape_and_cache(c["new_k"], c["new_v"], BF16, okc, ovc, cache_dt, c["new_slots"], None, ks, vs)
    ref = oracle.decode_attention(c["q"], BF16, okc, ovc, cache_dt, c["bt"], c["ctx"], scale, ks, vs)
    return ref, okc, ovc


CASES = [
    # name, ctx, hq, hkv, d, bs, cache, slot mode
    ("G2 D128 bf16", [1, 16, 17, 300, 1000, 64], 16, 8, 128, 16, BF16, "table"),
    ("G2 D128 fp8 scaled", [2, 15, 129, 700], 16, 8, 128, 16, FP8, "table"),
    ("G1 D128 bf16", [5, 77, 512], 8, 8, 128, 16, BF16, "table"),
    ("G4 D64 fp8", [31, 200, 9], 16, 4, 64, 16, FP8, "table"),
    ("G8 D128 bf16 bs32", [3, 65, 333], 16, 2, 128, 32, BF16, "table"),
    ("G2 D128 bf16 empty sequences", [0, 40, 0, 1, 90], 16, 8, 128, 16, BF16, "table"),
    ("G2 D128 bf16 skipped writes", [10, 40, 70, 33], 16, 8, 128, 16, BF16, "skip"),
    ("G2 D128 fp8 writes elsewhere", [10, 40, 70, 33], 16, 8, 128, 16, FP8, "elsewhere"),
    # fp8 caches run four KV heads per workgroup: six heads leave two waves idle,
    # three make a three-wave workgroup
    ("G2 D128 fp8 6 kv heads (idle waves)", [17, 300, 1, 129], 12, 6, 128, 16, FP8, "table"),
    ("G2 D128 fp8 3 kv heads", [64, 65, 500], 6, 3, 128, 16, FP8, "table"),
    ("G1 D128 fp8 bs32 skipped writes", [33, 2, 250], 8, 8, 128, 32, FP8, "skip"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_step_matches_write_then_attention(case):
    name, ctx, hq, hkv, d, bs, cdt, mode = case
    say(f"decode_step {name} B={len(ctx)}")
    c = make_step(zlib.crc32(name.encode()), ctx, hq, hkv, d, bs, cdt, slot_mode=mode)
    ks, vs = (0.05, 0.04) if cdt == FP8 else (None, None)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ref, okc, ovc = oracle_step(c, cdt, scale, ks, vs)
    for out_dt in (F32, BF16):
        out, gkc, gvc = gpu_step(c, cdt, scale, ks, vs, out_dt)
        assert np.array_equal(gkc.view(np.uint8), okc.view(np.uint8)), f"{name}: key cache"
        assert np.array_equal(gvc.view(np.uint8), ovc.view(np.uint8)), f"{name}: value cache"
        assert_attention_close(widen_out(out), ref, f"{name} out={'f32' if out_dt == F32 else 'bf16'}",
                               out_bf16=out_dt == BF16)


def test_full_b64_step_equals_separate_calls():
    """The batch-64 Qwen3-0.6B step: the one-call step leaves the caches
    bit-identical to reshape_and_cache followed by decode_attention on the GPU,
    and its output within the attention tolerance of theirs (the step takes the
    new token into the softmax after the cached positions, a different order of
    the same fp32 sums)."""
    m = pkv()
    w = workloads.qwen3_decode_b64()
    B, HQ, HKV, D, BS, NB = (w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size,
                             w.block_size, w.num_blocks)
    say(f"decode_step full size {w.name}")
    kc = workloads.device_normal((NB, BS, HKV, D), torch.bfloat16, "cuda", w.seed)
    vc = workloads.device_normal((NB, BS, HKV, D), torch.bfloat16, "cuda", w.seed + 1)
    q = workloads.device_normal((B, HQ, D), torch.bfloat16, "cuda", w.seed + 2)
    nk = workloads.device_normal((B, HKV, D), torch.bfloat16, "cuda", w.seed + 3)
    nv = workloads.device_normal((B, HKV, D), torch.bfloat16, "cuda", w.seed + 4)
    slots = torch.from_numpy(w.new_token_slots).cuda()
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.context_lens).cuda()
    kc2, vc2 = kc.clone(), vc.clone()
    out1 = torch.empty_like(q)
    m.decode_step(nk, nv, slots, out1, q, kc, vc, bt, cl, w.softmax_scale)
    out2 = torch.empty_like(q)
    m.reshape_and_cache(nk, nv, kc2, vc2, slots)
    m.decode_attention(out2, q, kc2, vc2, bt, cl, w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))
    assert_attention_close(widen_out(out1), widen_out(out2).astype(np.float64), "step vs separate calls",
                           out_bf16=True)


def test_step_in_a_hip_graph_replays_exactly():
    """Captured once, replayed five times with eager work and synchronisations in
    between; every replay's output equals the eager step's."""
    m = pkv()
    say("decode_step graph capture")
    c = make_step(5150, [33, 400, 1000, 64, 7], 16, 8, 128, 16, BF16)
    dk, dv = to_dev(c["kc"], BF16), to_dev(c["vc"], BF16)
    q = to_dev(c["q"], BF16)
    nk, nv = to_dev(c["new_k"], BF16), to_dev(c["new_v"], BF16)
    slots = torch.from_numpy(c["new_slots"]).cuda()
    bt = torch.from_numpy(c["bt"]).cuda()
    cl = torch.from_numpy(c["ctx"]).cuda()
    ws = torch.empty(m.decode_attention_workspace_size(5, 16, 8, 128, c["bt"].shape[1], 16),
                     dtype=torch.uint8, device="cuda")
    eager = torch.empty_like(q)
    m.decode_step(nk, nv, slots, eager, q, dk, dv, bt, cl, 0.088, workspace=ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(q)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.decode_step(nk, nv, slots, out, q, dk, dv, bt, cl, 0.088, workspace=ws)  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        m.decode_step(nk, nv, slots, out, q, dk, dv, bt, cl, 0.088, workspace=ws)
    for i in range(5):
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        del junk
