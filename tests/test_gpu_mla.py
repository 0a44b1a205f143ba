"""GPU parity of MLA decode over a latent paged cache (absorbed weights on the
GPU) against the oracle, which writes K and V out from the latent as the page
defines them (reading R13).

Tolerance: the decode bound 2e-3 + 2e-3*|o| (fp32 outputs; bf16 outputs get
half a bf16 ulp more). The GPU's extra steps stay far inside it: the absorbed
query and the probabilities enter the matrix cores as bf16 hi + lo pairs (each
within 2^-17 relative of the fp32 value), every product is exact in fp32 and
the sums run in fp32 over at most 576 terms per step.

Cases: ragged contexts around the 32-position tile and the 256-position piece,
with and without a RoPE part, block sizes 1, 16, 48, 64, other qk / v widths,
empty contexts, bad table entries and clamped lengths, NaN in every slot no
sequence owns, bit-identical output under block relabelling, the full batch-64
workload on every sequence (one head each), and a decode step whose latent rows
are first written by concat_and_cache_mla_k, and 300 repeated full-size calls
that must agree bit for bit."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import assert_attention_close, say, to_dev, to_host, widen_out

pytestmark = pytest.mark.gpu

BF16, F32 = oracle.BF16, oracle.F32
NAN_BF16 = 0x7FC0
H, DC = 16, 512


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def pkv():
    import paged_kv_cache_304_amd as m
    return m


def weight_bits(rng, shape):
    return workloads.normal_bf16_bits(rng, shape, std=1.0 / np.sqrt(DC))


def make_case(seed, ctx, R=64, QK=128, DV=128, bs=16, spare=4, width=None):
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    nblk = [-(-int(c) // bs) for c in ctx]
    nb = sum(nblk) + spare
    W = width or max(max(nblk), 1)
    bt = workloads.deal_block_tables(rng.permutation(nb).astype(np.int32), ctx, bs, W)
    cache = workloads.normal_bf16_bits(rng, (nb, bs, DC + R))
    owned = np.zeros((nb, bs), dtype=bool)
    for b, c in enumerate(ctx):
        pos = np.arange(int(c))
        owned[bt[b, pos // bs], pos % bs] = True
    cache[~owned] = NAN_BF16
    return dict(ctx=ctx, bt=bt, cache=cache, R=R, QK=QK, DV=DV,
                q_nope=workloads.normal_bf16_bits(rng, (len(ctx), H, QK)),
                q_rope=workloads.normal_bf16_bits(rng, (len(ctx), H, R)) if R else None,
                w_uk=weight_bits(rng, (DC, H * QK)), w_uv=weight_bits(rng, (DC, H * DV)),
                scale=float(np.float32(1.0 / np.sqrt(QK + R))))


def gpu_mla(c, out_dt=F32, **over):
    m = pkv()
    c = dict(c, **over)
    B = len(c["ctx"])
    out = torch.full((B, H, c["DV"]), float("nan"), device="cuda",
                     dtype=torch.float32 if out_dt == F32 else torch.bfloat16)
    m.mla_decode_attention(out, to_dev(c["q_nope"], BF16),
                           None if c["q_rope"] is None else to_dev(c["q_rope"], BF16),
                           to_dev(c["w_uk"], BF16), to_dev(c["w_uv"], BF16), to_dev(c["cache"], BF16),
                           torch.from_numpy(c["bt"]).cuda(), torch.from_numpy(c["ctx"]).cuda(), c["scale"])
    torch.cuda.synchronize()
    return widen_out(out)


def oracle_mla(c, **over):
    c = dict(c, **over)
    return oracle.mla_decode(c["q_nope"], c["q_rope"], c["w_uk"], c["w_uv"], c["cache"], c["bt"], c["ctx"],
                             c["scale"])


CASES = [
    # name, ctx, rope, qk, v, block size
    ("R64 ragged around tiles and pieces", [1, 31, 32, 33, 255, 256, 257, 700, 0], 64, 128, 128, 16),
    ("no RoPE part", [5, 300, 64], 0, 128, 128, 16),
    ("bs64 qk64 v64", [100, 513], 64, 64, 64, 64),
    ("bs1", [17, 300], 64, 128, 128, 1),
    ("bs48", [250, 49, 97], 64, 128, 128, 48),
    ("qk256 v256", [90, 260], 64, 256, 256, 16),
    ("qk32 v32 no RoPE", [40], 0, 32, 32, 16),
    # narrow values: each merge thread's slice of W_UV is 2 (v8) or 4 (v16) latent rows
    ("qk16 v8", [70, 3, 300], 64, 16, 8, 16),
    ("qk24 v16", [129, 1], 0, 24, 16, 16),
    # more than 64 sequences: the split's segment set-up searches the tile plan
    ("B65 one past a single round of set-up loads", [(37 * i) % 200 + 1 for i in range(65)], 64, 128, 128, 16),
    # on 256 compute units the first workgroup's five units are sequence 0's
    # query and tile, sequence 71's query and tile and sequence 72's query:
    # its tiles lie 71 entries apart and its list of segments is refilled
    ("B73 a refilled segment list", [1] + [0] * 70 + [1, 40000], 64, 128, 128, 16),
    # more than 256 sequences: each thread of the tile plan sums a run of two
    ("B300 two sequences per plan thread", [(17 * i) % 90 + (i % 7 != 3) for i in range(300)], 64, 128, 128, 16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mla_matches_oracle(case):
    name, ctx, R, QK, DV, bs = case
    say(f"mla_decode {name} ctx={ctx} R={R} qk={QK} v={DV} bs={bs}")
    c = make_case(zlib.crc32(name.encode()), ctx, R, QK, DV, bs)
    ref = oracle_mla(c)
    for out_dt in (F32, BF16):
        got = gpu_mla(c, out_dt)
        assert_attention_close(got, ref, f"{name} out={'f32' if out_dt == F32 else 'bf16'}",
                               out_bf16=out_dt == BF16)


def test_bad_table_entries_and_clamped_lengths():
    say("mla_decode bad table entries")
    c = make_case(91, [90, 64, 48], width=6)
    bt = c["bt"].copy()
    nb = c["cache"].shape[0]
    bt[0, 2] = nb + 3
    bt[1, 0] = -7
    ctx = np.array([90, 64, 9999], dtype=np.int32)   # sequence 2 clamped to 96 positions
    bt[2, 3:] = nb + 100
    ref = oracle_mla(c, bt=bt, ctx=ctx)
    assert_attention_close(gpu_mla(c, bt=bt, ctx=ctx), ref, "bad entries", out_bf16=False)


def test_block_relabelling_is_bit_identical():
    say("mla_decode block relabelling")
    c = make_case(33, [300, 1234, 64], spare=20)
    a = gpu_mla(c)
    perm = np.random.default_rng(1).permutation(c["cache"].shape[0])
    cache2 = np.empty_like(c["cache"])
    cache2[perm] = c["cache"]
    bt2 = np.where(c["bt"] >= 0, perm[np.maximum(c["bt"], 0)], -1).astype(np.int32)
    b = gpu_mla(c, cache=cache2, bt=bt2)
    assert np.array_equal(a, b)


def full_size_tensors(w):
    B, R, DCR = w["num_seqs"], w["rope_dim"], w["kv_lora_rank"] + w["rope_dim"]
    s = w["seed"]
    cache = workloads.device_normal((w["num_blocks"], w["block_size"], DCR), torch.bfloat16, "cuda", s)
    q_nope = workloads.device_normal((B, H, w["qk_nope_dim"]), torch.bfloat16, "cuda", s + 1)
    q_rope = workloads.device_normal((B, H, R), torch.bfloat16, "cuda", s + 2)
    w_uk = workloads.device_normal((DC, H * w["qk_nope_dim"]), torch.bfloat16, "cuda", s + 3, std=w["w_std"])
    w_uv = workloads.device_normal((DC, H * w["v_dim"]), torch.bfloat16, "cuda", s + 4, std=w["w_std"])
    return cache, q_nope, q_rope, w_uk, w_uv


def test_full_size_mla_batch_every_sequence():
    """The batch-64 MLA workload in the launch the benchmark times (bf16 out),
    and again with an fp32 output at the plain bound: every sequence against the
    oracle on one of its heads (head b % 16, so each head is checked on four
    sequences). Heads are independent, so head h of sequences b = h (mod 16) is
    a one-head MLA problem of its own (W_UK and W_UV columns of head h) that the
    oracle solves at 1/16 of the full cost."""
    m = pkv()
    w = workloads.mla_decode_b64()
    say(f"mla_decode full size {w['name']}")
    cache, q_nope, q_rope, w_uk, w_uv = full_size_tensors(w)
    bt, ctx = w["block_tables"], w["context_lens"]
    outs = {}
    for dt in (torch.bfloat16, torch.float32):
        out = torch.empty((w["num_seqs"], H, w["v_dim"]), dtype=dt, device="cuda")
        m.mla_decode_attention(out, q_nope, q_rope, w_uk, w_uv, cache, torch.from_numpy(bt).cuda(),
                               torch.from_numpy(ctx).cuda(), w["softmax_scale"])
        torch.cuda.synchronize()
        outs[dt] = widen_out(out)
    ch = to_host(cache, BF16)
    qn, qr, wk, wv = (to_host(t, BF16) for t in (q_nope, q_rope, w_uk, w_uv))
    QK, DV = w["qk_nope_dim"], w["v_dim"]
    for h in range(H):
        sel = np.arange(h, w["num_seqs"], H)
        ref = oracle.mla_decode(np.ascontiguousarray(qn[sel, h:h + 1]), np.ascontiguousarray(qr[sel, h:h + 1]),
                                np.ascontiguousarray(wk[:, h * QK:(h + 1) * QK]),
                                np.ascontiguousarray(wv[:, h * DV:(h + 1) * DV]), ch,
                                np.ascontiguousarray(bt[sel]), np.ascontiguousarray(ctx[sel]), w["softmax_scale"])
        for dt, name in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
            assert_attention_close(outs[dt][sel, h:h + 1], ref, f"{w['name']} head {h} sequences {list(sel)} out={name}",
                                   out_bf16=dt == torch.bfloat16)


def test_mla_decode_step_writes_latent_rows_then_attends():
    """The new token's latent row (c ++ k_rope, one 'head') goes into the cache
    with concat_and_cache_mla_k, then MLA decode reads it back: the cache
    bit-exact against the oracle's concat + write, the output against the
    oracle's MLA decode on that cache."""
    m = pkv()
    say("mla decode step")
    c = make_case(4242, [40, 1, 300, 17])
    rng = np.random.default_rng(7)
    B, R, QK = len(c["ctx"]), c["R"], c["QK"]
    bs = c["cache"].shape[1]
    new_c = workloads.normal_bf16_bits(rng, (B, 1, DC))
    new_r = workloads.normal_bf16_bits(rng, (B, 1, R))
    pos = c["ctx"].astype(np.int64) - 1
    slots = workloads.slots_for_positions(c["bt"], np.arange(B), pos, bs)
    cache = c["cache"].copy()
    for b in range(B):                       # the new positions hold NaN until written
        cache[slots[b] // bs, slots[b] % bs] = NAN_BF16
    ocache = cache.copy()
    k = np.zeros((B, 1, DC + R), dtype=np.float32)
    oracle.concat_and_cast(k, oracle.F32, new_c, BF16, new_r, BF16)
    oracle.reshape_and_cache(k, None, oracle.F32, ocache.reshape(-1, bs, 1, DC + R), None, BF16, slots)
    ref = oracle_mla(c, cache=ocache)
    dcache = to_dev(cache, BF16)
    m.concat_and_cache_mla_k(to_dev(new_c, BF16), to_dev(new_r, BF16), dcache.view(-1, bs, 1, DC + R),
                             torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_host(dcache, BF16), ocache), "latent cache"
    got = gpu_mla(c, cache=to_host(dcache, BF16))
    assert_attention_close(got, ref, "mla step", out_bf16=False)


@pytest.mark.parametrize("R", [64, 0])
def test_mla_decode_step_entry_writes_then_attends_in_one_call(R):
    """pa_mla_decode_step: the cache bit-exact against the oracle's concat + write
    (a negative slot and one past the pool write nothing), the output against
    the oracle's MLA decode on that cache, and bit-identical to the two calls it
    replaces (concat_and_cache_mla_k, then mla_decode_attention). 520 sequences:
    more rows than the absorb launch's writing waves (508)."""
    m = pkv()
    ctx = [40, 1, 300, 17, 64] + [1 + (i * 7) % 12 for i in range(515)]
    say(f"mla decode step entry R={R} B={len(ctx)}")
    c = make_case(4243 + R, ctx, R=R)
    rng = np.random.default_rng(8 + R)
    B = len(c["ctx"])
    bs = c["cache"].shape[1]
    nb = c["cache"].shape[0]
    new_c = workloads.normal_bf16_bits(rng, (B, DC))
    new_r = workloads.normal_bf16_bits(rng, (B, R)) if R else None
    pos = c["ctx"].astype(np.int64) - 1
    slots = workloads.slots_for_positions(c["bt"], np.arange(B), pos, bs)
    cache = c["cache"].copy()
    for b in range(B):
        if b not in (2, 3):                  # the new positions hold NaN until written
            cache[slots[b] // bs, slots[b] % bs] = NAN_BF16
    slots[2] = -1                            # skipped: its last position keeps its row
    slots[3] = nb * bs                       # past the pool: skipped too
    ocache = cache.copy()
    k = np.zeros((B, 1, DC + R), dtype=np.float32)
    oracle.concat_and_cast(k, oracle.F32, new_c[:, None, :], BF16,
                           new_r[:, None, :] if R else np.zeros((B, 1, 0), dtype=np.uint16), BF16)
    oracle.reshape_and_cache(k, None, oracle.F32, ocache.reshape(-1, bs, 1, DC + R), None, BF16, slots)
    ref = oracle_mla(c, cache=ocache)

    dslots = torch.from_numpy(slots).cuda()
    args = lambda dc, out: (out, to_dev(c["q_nope"], BF16), None if R == 0 else to_dev(c["q_rope"], BF16),
                            to_dev(c["w_uk"], BF16), to_dev(c["w_uv"], BF16), dc,
                            torch.from_numpy(c["bt"]).cuda(), torch.from_numpy(c["ctx"]).cuda(), c["scale"])
    dcache = to_dev(cache, BF16)
    out = torch.full((B, H, c["DV"]), float("nan"), device="cuda")
    m.mla_decode_step(to_dev(new_c, BF16), None if R == 0 else to_dev(new_r, BF16), dslots, *args(dcache, out))
    # the two calls it replaces
    dcache2 = to_dev(cache, BF16)
    out2 = torch.full_like(out, float("nan"))
    if R:
        m.concat_and_cache_mla_k(to_dev(new_c, BF16)[:, None, :], to_dev(new_r, BF16)[:, None, :],
                                 dcache2.view(-1, bs, 1, DC + R), dslots)
    m.mla_decode_attention(*args(dcache2, out2))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(dcache, BF16), ocache), "latent cache"
    assert_attention_close(widen_out(out), ref, "mla step entry", out_bf16=False)
    if R:
        # (bit patterns: slots no sequence owns hold NaN)
        assert torch.equal(dcache.view(torch.int16), dcache2.view(torch.int16)), "fused step's cache differs"
        assert torch.equal(out.view(torch.int32), out2.view(torch.int32)), "fused step's output differs"


def test_mla_in_a_hip_graph_replays_exactly():
    """Captured once (workspace supplied), replayed four times with new queries
    and eager work in between; every replay equals an eager call."""
    m = pkv()
    say("mla_decode graph capture")
    c = make_case(515, [300, 1, 700, 64])
    B = len(c["ctx"])
    qn, qr = to_dev(c["q_nope"], BF16), to_dev(c["q_rope"], BF16)
    wk, wv, cache = to_dev(c["w_uk"], BF16), to_dev(c["w_uv"], BF16), to_dev(c["cache"], BF16)
    bt, cl = torch.from_numpy(c["bt"]).cuda(), torch.from_numpy(c["ctx"]).cuda()
    ws = torch.empty(m.mla_decode_workspace_size(B, H, c["QK"], c["R"], DC, c["DV"], c["bt"].shape[1],
                                                 c["cache"].shape[1]), dtype=torch.uint8, device="cuda")
    out = torch.zeros((B, H, c["DV"]), dtype=torch.float32, device="cuda")
    eager = torch.zeros_like(out)
    call = lambda o: m.mla_decode_attention(o, qn, qr, wk, wv, cache, bt, cl, c["scale"], workspace=ws)  # noqa: E731
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    rng = np.random.default_rng(2)
    for i in range(4):
        qn.copy_(to_dev(workloads.normal_bf16_bits(rng, c["q_nope"].shape), BF16))
        qr.copy_(to_dev(workloads.normal_bf16_bits(rng, c["q_rope"].shape), BF16))
        out.zero_()
        junk = torch.randn(1 << 18, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(eager)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        del junk


def test_mla_decode_step_in_a_hip_graph_replays_exactly():
    """The one-call step captured once, replayed four times with new latent rows
    and queries and eager work in between: every replay leaves the new rows in
    their slots and equals an eager step."""
    m = pkv()
    say("mla_decode_step graph capture")
    c = make_case(516, [300, 1, 700, 64])
    B, R, bs = len(c["ctx"]), c["R"], c["cache"].shape[1]
    qn, qr = to_dev(c["q_nope"], BF16), to_dev(c["q_rope"], BF16)
    wk, wv, cache = to_dev(c["w_uk"], BF16), to_dev(c["w_uv"], BF16), to_dev(c["cache"], BF16)
    bt, cl = torch.from_numpy(c["bt"]).cuda(), torch.from_numpy(c["ctx"]).cuda()
    slots = workloads.slots_for_positions(c["bt"], np.arange(B), c["ctx"].astype(np.int64) - 1, bs)
    dslots = torch.from_numpy(slots).cuda()
    rng = np.random.default_rng(3)
    nc = to_dev(workloads.normal_bf16_bits(rng, (B, DC)), BF16)
    nr = to_dev(workloads.normal_bf16_bits(rng, (B, R)), BF16)
    ws = torch.empty(m.mla_decode_workspace_size(B, H, c["QK"], R, DC, c["DV"], c["bt"].shape[1], bs),
                     dtype=torch.uint8, device="cuda")
    out = torch.zeros((B, H, c["DV"]), dtype=torch.float32, device="cuda")
    eager = torch.zeros_like(out)
    step = lambda o: m.mla_decode_step(nc, nr, dslots, o, qn, qr, wk, wv, cache, bt, cl, c["scale"],  # noqa: E731
                                       workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    flat = cache.view(-1, DC + R)
    for i in range(4):
        nc.copy_(to_dev(workloads.normal_bf16_bits(rng, (B, DC)), BF16))
        nr.copy_(to_dev(workloads.normal_bf16_bits(rng, (B, R)), BF16))
        qn.copy_(to_dev(workloads.normal_bf16_bits(rng, c["q_nope"].shape), BF16))
        out.zero_()
        junk = torch.randn(1 << 18, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rows = flat[dslots]
        assert torch.equal(rows.view(torch.int16), torch.cat([nc, nr], dim=1).view(torch.int16)), f"rows {i}"
        step(eager)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        del junk


def test_repeated_full_size_calls_are_identical_and_finite():
    """300 calls of the batch-64 workload back to back, ten outputs in flight
    at a time: the split kernel's waves hand work to each other at their own
    pace in every call, and the result must not depend on it -- every output
    bit-identical to the first and finite (a hand-off wait that ran past its
    bound would make the call's outputs NaN)."""
    m = pkv()
    w = workloads.mla_decode_b64()
    say(f"mla_decode repeated {w['name']}")
    cache, q_nope, q_rope, w_uk, w_uv = full_size_tensors(w)
    bt = torch.from_numpy(w["block_tables"]).cuda()
    ctx = torch.from_numpy(w["context_lens"]).cuda()
    ws = torch.empty(m.mla_decode_workspace_size(w["num_seqs"], H, w["qk_nope_dim"], w["rope_dim"], DC, w["v_dim"],
                                                 bt.shape[1], w["block_size"]), dtype=torch.uint8, device="cuda")
    outs = torch.empty((10, w["num_seqs"], H, w["v_dim"]), dtype=torch.float32, device="cuda")
    first = None
    for rnd in range(30):
        for i in range(10):
            m.mla_decode_attention(outs[i], q_nope, q_rope, w_uk, w_uv, cache, bt, ctx, w["softmax_scale"],
                                   workspace=ws)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(outs).all()), f"round {rnd}: non-finite output"
        if first is None:
            first = outs[0].clone()
        for i in range(10):
            assert torch.equal(outs[i], first), f"round {rnd} call {i} differs from the first call"
