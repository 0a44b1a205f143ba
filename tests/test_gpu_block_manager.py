"""The block manager feeding the GPU path, step by step, against the oracle.

An engine-style run on one layer's caches: prefill chunks, decode steps,
mixed steps, releases and re-use of freed blocks, a refused step, steps
launched at fixed padded sizes. Each step's metadata is planned by the native
manager, uploaded with its one copy, and read by the kernels from device
memory; the oracle plans the same step with its own block pool and runs its
own write and attention. Checked every step: the uploaded metadata against the
oracle's arrays (bit-exact), both whole caches (bit-exact), the attention
output within the attention tolerance -- with the uploads on a copy stream
overlapping the previous step's kernels, and on the compute stream. Also: the
upload plus decode step
captured in a HIP graph and replayed for later steps, each replay against the
oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.block_pool import BlockPool, NoSpace
from parity_util import (assert_attention_close, say, to_dev, to_host,
                         widen_out)

pytestmark = pytest.mark.gpu

BF16 = oracle.BF16
NAN_BF16 = 0x7FC0
HQ, HKV, D, BS = 16, 8, 128, 16
NB, S, W, B_MAX, T_MAX = 120, 8, 40, 6, 700
SCALE = float(np.float32(1.0 / np.sqrt(D)))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def pkv():
    import paged_kv_cache_304_amd as m
    return m


class Engine:
    """Device caches driven through the native manager, host caches through the oracle pool."""

    def __init__(self, seed, overlap=True):
        m = pkv()
        self.m = m
        self.rng = np.random.default_rng(seed)
        self.bm = m.BlockManager(NB, BS, S, W, B_MAX, T_MAX)
        self.stager = m.StepStager(self.bm, overlap=overlap)
        self.pool = BlockPool(NB, BS, W)
        self.okc = np.full((NB, BS, HKV, D), NAN_BF16, dtype=np.uint16)
        self.ovc = self.okc.copy()
        self.kc = to_dev(self.okc, BF16)
        self.vc = to_dev(self.ovc, BF16)
        self.ws = torch.empty(m.decode_attention_workspace_size(B_MAX, HQ, HKV, D, W, BS),
                              dtype=torch.uint8, device="cuda")

    def release(self, s):
        self.bm.release(s)
        self.pool.release(s)

    def inputs(self, T, real):
        nk = np.zeros((T, HKV, D), dtype=np.uint16)
        nv = np.zeros_like(nk)
        q = np.zeros((T, HQ, D), dtype=np.uint16)
        nk[:real] = workloads.normal_bf16_bits(self.rng, (real, HKV, D))
        nv[:real] = workloads.normal_bf16_bits(self.rng, (real, HKV, D))
        q[:real] = workloads.normal_bf16_bits(self.rng, (real, HQ, D))
        return nk, nv, q

    def step(self, seqs, num, pad=False, what=""):
        say(f"engine step {what}: seqs={list(seqs)} num={list(num)} pad={pad}")
        m = self.m
        ps, pt = (B_MAX, T_MAX) if pad else (None, None)
        decode = all(n == 1 for n in num)
        if decode and pad:
            pt = B_MAX                      # one token per row: token i belongs to row i
        sm, bt, cl, cu = self.pool.step_arrays(seqs, num, W, ps, pt)
        dev = self.stager.step(seqs, num, ps, pt)
        rows, T = dev.num_seqs, dev.num_tokens
        # the metadata the kernels will read, as uploaded
        assert np.array_equal(dev.slot_mapping.cpu().numpy(), sm), f"{what}: slot_mapping"
        assert np.array_equal(dev.block_tables.cpu().numpy(), bt), f"{what}: block_tables"
        assert np.array_equal(dev.context_lens.cpu().numpy(), cl), f"{what}: context_lens"
        assert np.array_equal(dev.cu_seqlens_q.cpu().numpy(), cu), f"{what}: cu_seqlens_q"
        nk, nv, q = self.inputs(T, int(sum(num)))
        dq = to_dev(q, BF16)
        out = torch.full(dq.shape, float("nan"), dtype=torch.float32, device="cuda")
        oracle.reshape_and_cache(nk, nv, BF16, self.okc, self.ovc, BF16, sm, None)
        if decode:
            m.decode_step(to_dev(nk, BF16), to_dev(nv, BF16), dev.slot_mapping, out, dq, self.kc,
                          self.vc, dev.block_tables, dev.context_lens, SCALE, workspace=self.ws)
            ref = oracle.decode_attention(q, BF16, self.okc, self.ovc, BF16, bt, cl, SCALE)
        else:
            m.reshape_and_cache(to_dev(nk, BF16), to_dev(nv, BF16), self.kc, self.vc, dev.slot_mapping)
            m.prefill_attention(out, dq, dev.cu_seqlens_q, self.kc, self.vc, dev.block_tables,
                                dev.context_lens, SCALE)
            real = int(cu[-1])                  # the oracle takes only the rows sequences own
            ref = oracle.prefill_attention(q[:real], BF16, cu, self.okc, self.ovc, BF16, bt, cl, SCALE)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(self.kc, BF16), self.okc), f"{what}: key cache"
        assert np.array_equal(to_host(self.vc, BF16), self.ovc), f"{what}: value cache"
        got = widen_out(out)
        if decode:
            assert_attention_close(got[:rows], ref[:rows], what, out_bf16=False)
        else:
            assert_attention_close(got[:real], ref, what, out_bf16=False)
            assert np.all(np.isnan(got[real:])), f"{what}: padding rows were written"
        return rows, T


# An engine's run: ("step", seqs, new tokens, padded, label), ("release", seq),
# ("refuse", seqs, new tokens) -- a step that needs more blocks than are free.
SCRIPT = [
    ("step", [0, 1, 2], [100, 37, 250], False, "prefill three prompts"),
    ("step", [0, 1, 2], [1, 1, 1], False, "decode"),
    ("step", [3, 0], [300, 1], False, "mixed: a new prompt and one decode token"),
    ("release", 1),
    ("step", [4], [64], False, "new prompt re-using freed blocks"),
    ("step", [0, 2, 3, 4], [1, 1, 1, 1], True, "padded decode 0"),
    ("step", [0, 2, 3, 4], [1, 1, 1, 1], True, "padded decode 1"),
    ("step", [0, 2, 3, 4], [1, 1, 1, 1], True, "padded decode 2"),
    ("step", [2, 5], [129, 17], True, "padded chunks"),
    ("step", [6], [W * BS], False, "a prompt filling its whole table"),
    ("refuse", [7], [400]),
    ("release", 0),
    ("release", 3),
    ("release", 6),
    ("step", [7, 2], [500, 1], False, "large chunk after releases"),
    ("step", [2, 4, 5, 7], [1, 1, 1, 1], False, "decode after re-use"),
]


@pytest.mark.parametrize("overlap", [True, False], ids=["copy-stream", "one-stream"])
def test_engine_run_matches_the_oracle(overlap):
    e = Engine(2024, overlap)
    for act in SCRIPT:
        if act[0] == "step":
            e.step(act[1], act[2], pad=act[3], what=act[4])
        elif act[0] == "release":
            e.release(act[1])
        else:
            free = e.bm.free_blocks
            with pytest.raises(e.m.PagedKVError) as ei:
                e.bm.plan_host(act[1], act[2])
            assert ei.value.status == e.m._lib.PA_ENOSPACE and e.bm.free_blocks == free
            with pytest.raises(NoSpace):
                e.pool.step(act[1], act[2])


def test_upload_and_decode_step_replay_in_a_graph():
    """Capture (upload + decode step) at fixed padded sizes once; each later
    step plans into the same pinned blob and replays the graph."""
    m = pkv()
    say("block manager graph replay")
    rng = np.random.default_rng(7)
    bm = m.BlockManager(NB, BS, S, W, B_MAX, T_MAX)
    st = m.StepStager(bm, depth=1)
    pool = BlockPool(NB, BS, W)
    okc = workloads.normal_bf16_bits(rng, (NB, BS, HKV, D))
    ovc = workloads.normal_bf16_bits(rng, (NB, BS, HKV, D))
    kc, vc = to_dev(okc, BF16), to_dev(ovc, BF16)
    seqs = [0, 1, 2, 3]
    lens = [40, 77, 300, 5]
    # prompts: written directly, no attention needed
    dev = st.step(seqs, lens)
    sm, _, _, _ = pool.step_arrays(seqs, lens, W)
    T = sum(lens)
    k0 = workloads.normal_bf16_bits(rng, (T, HKV, D))
    v0 = workloads.normal_bf16_bits(rng, (T, HKV, D))
    m.reshape_and_cache(to_dev(k0, BF16), to_dev(v0, BF16), kc, vc, dev.slot_mapping)
    oracle.reshape_and_cache(k0, v0, BF16, okc, ovc, BF16, sm, None)
    torch.cuda.synchronize()

    nk = torch.empty((B_MAX, HKV, D), dtype=torch.bfloat16, device="cuda")
    nv = torch.empty_like(nk)
    q = torch.empty((B_MAX, HQ, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(m.decode_attention_workspace_size(B_MAX, HQ, HKV, D, W, BS), dtype=torch.uint8,
                     device="cuda")
    host = st.host[0]
    lay = bm.layout

    def body():
        m._lib.check(m._lib.lib.pa_bm_upload(bm._h, host.data_ptr(), st.dev.data_ptr(), B_MAX,
                                             torch.cuda.current_stream().cuda_stream))
        d = st.dev
        slots = d[lay.slot_mapping:lay.slot_mapping + 8 * B_MAX].view(torch.int64)
        bt = d[lay.block_tables:lay.block_tables + 4 * B_MAX * W].view(torch.int32).view(B_MAX, W)
        cl = d[lay.context_lens:lay.context_lens + 4 * B_MAX].view(torch.int32)
        m.decode_step(nk, nv, slots, out, q, kc, vc, bt, cl, SCALE, workspace=ws)

    def plan_and_inputs():
        bm.plan_into(host.data_ptr(), host.numel(), seqs, [1] * len(seqs), B_MAX, B_MAX)
        sm, bt, cl, _ = pool.step_arrays(seqs, [1] * len(seqs), W, B_MAX, B_MAX)
        a = np.zeros((B_MAX, HKV, D), dtype=np.uint16)
        b = np.zeros_like(a)
        qq = np.zeros((B_MAX, HQ, D), dtype=np.uint16)
        a[:4] = workloads.normal_bf16_bits(rng, (4, HKV, D))
        b[:4] = workloads.normal_bf16_bits(rng, (4, HKV, D))
        qq[:4] = workloads.normal_bf16_bits(rng, (4, HQ, D))
        nk.copy_(to_dev(a, BF16))
        nv.copy_(to_dev(b, BF16))
        q.copy_(to_dev(qq, BF16))
        oracle.reshape_and_cache(a, b, BF16, okc, ovc, BF16, sm, None)
        return oracle.decode_attention(qq, BF16, okc, ovc, BF16, bt, cl, SCALE)

    ref = plan_and_inputs()                      # step 1, eager (also warms up)
    body()
    torch.cuda.synchronize()
    assert_attention_close(widen_out(out)[:4], ref[:4], "eager step", out_bf16=True)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        body()
    torch.cuda.synchronize()
    # capture enqueued nothing: the caches still hold step 1's state
    assert np.array_equal(to_host(kc, BF16), okc)
    for i in range(4):
        ref = plan_and_inputs()
        junk = torch.randn(1 << 18, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(kc, BF16), okc), f"replay {i}: key cache"
        assert np.array_equal(to_host(vc, BF16), ovc), f"replay {i}: value cache"
        assert_attention_close(widen_out(out)[:4], ref[:4], f"replay {i}", out_bf16=True)
        del junk
