"""PA_CHECK=1: every entry point copies its device-resident metadata to the host
and validates it before launching. Valid metadata runs exactly as without the
check; metadata the kernels would skip silently (slots outside the SWA table or
the pool, table entries outside the pool, lengths past the table) or could not
handle at all (two tokens writing one slot, a chunk longer than its context,
packed query offsets going backwards) is refused with PA_EINVAL, and nothing is
launched."""
import numpy as np
import pytest
import torch

from parity_util import say

pytestmark = pytest.mark.gpu

NB, BS = 16, 16


@pytest.fixture
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_304_amd as m
    return m


@pytest.fixture
def checked(monkeypatch):
    monkeypatch.setenv("PA_CHECK", "1")
    return monkeypatch


def randn(*shape, seed=0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(*shape, generator=g, device="cuda").to(torch.bfloat16)


def refused(m, fn, text):
    with pytest.raises(m.PagedKVError) as ei:
        fn()
    assert ei.value.status == 1 and "PA_CHECK" in str(ei.value) and text in str(ei.value), str(ei.value)


# ------------------------------------------------------------------ cache writes
def write_case(T=8, H=2, D=64):
    key, val = randn(T, H, D, seed=1), randn(T, H, D, seed=2)
    kc = torch.full((NB, BS, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    vc = kc.clone()
    slots = torch.arange(T, dtype=torch.int64, device="cuda") * 3
    slots[1] = -1  # skipped, allowed
    return key, val, kc, vc, slots


def test_valid_write_runs_as_without_the_check(m, checked):
    say("PA_CHECK valid reshape_and_cache")
    key, val, kc, vc, slots = write_case()
    kc2, vc2 = kc.clone(), vc.clone()
    m.reshape_and_cache(key, val, kc, vc, slots)
    checked.delenv("PA_CHECK")
    m.reshape_and_cache(key, val, kc2, vc2, slots)
    torch.cuda.synchronize()
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2)


@pytest.mark.parametrize("case", ["past the pool", "one slot twice", "past the SWA table", "SWA to one slot"])
def test_bad_write_metadata_is_refused_and_nothing_written(m, checked, case):
    say(f"PA_CHECK reshape_and_cache: {case}")
    key, val, kc, vc, slots = write_case()
    before = kc.clone()
    swa = None
    if case == "past the pool":
        slots[3], text = NB * BS, "past the pool"
    elif case == "one slot twice":
        slots[5], text = slots[2].item(), "both write slot"
    elif case == "past the SWA table":
        swa = torch.arange(20, dtype=torch.int64, device="cuda")
        slots[4], text = 20, "past the SWA table"
    else:
        swa = torch.arange(30, dtype=torch.int64, device="cuda")
        swa[int(slots[6])] = int(slots[0])  # tokens 0 and 6 land on one final slot
        text = "both write slot"
    refused(m, lambda: m.reshape_and_cache(key, val, kc, vc, slots, swa), text)
    torch.cuda.synchronize()
    assert torch.equal(kc, before)


def test_fused_mla_k_write_is_checked(m, checked):
    say("PA_CHECK concat_and_cache_mla_k")
    T, H, nope, rope = 6, 2, 64, 32
    kn, kr = randn(T, H, nope, seed=3), randn(T, 1, rope, seed=4)
    cache = torch.zeros((NB, BS, H, nope + rope), dtype=torch.bfloat16, device="cuda")
    slots = torch.arange(T, dtype=torch.int64, device="cuda") * 5
    m.concat_and_cache_mla_k(kn, kr, cache, slots)
    slots[2] = slots[4]
    refused(m, lambda: m.concat_and_cache_mla_k(kn, kr, cache, slots), "both write slot")


# ------------------------------------------------------------------ attention
def decode_case(ctx=(5, 40, 0), HQ=4, HKV=2, D=64, W=4):
    rng = np.random.default_rng(11)
    bt = np.full((len(ctx), W), -1, dtype=np.int32)
    perm = rng.permutation(NB).astype(np.int32)
    k = 0
    for b, c in enumerate(ctx):
        n = -(-c // BS)
        bt[b, :n] = perm[k:k + n]
        k += n
    kc, vc = randn(NB, BS, HKV, D, seed=5), randn(NB, BS, HKV, D, seed=6)
    q = randn(len(ctx), HQ, D, seed=7)
    return (q, kc, vc, torch.from_numpy(bt).cuda(), torch.tensor(ctx, dtype=torch.int32, device="cuda"))


def test_valid_decode_runs_as_without_the_check(m, checked):
    say("PA_CHECK valid decode_attention")
    q, kc, vc, bt, cl = decode_case()
    a = m.decode_attention(torch.empty_like(q), q, kc, vc, bt, cl, 0.125)
    checked.delenv("PA_CHECK")
    b = m.decode_attention(torch.empty_like(q), q, kc, vc, bt, cl, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("case", ["entry outside the pool", "length past the table", "negative length"])
def test_bad_decode_metadata_is_refused(m, checked, case):
    say(f"PA_CHECK decode_attention: {case}")
    q, kc, vc, bt, cl = decode_case()
    if case == "entry outside the pool":
        bt[1, 2], text = NB, "outside the pool"
    elif case == "length past the table":
        cl[0], text = 4 * BS + 1, "context length"
    else:
        cl[2], text = -1, "context length"
    out = torch.full_like(q, 3.0)
    refused(m, lambda: m.decode_attention(out, q, kc, vc, bt, cl, 0.125), text)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


def test_decode_step_checks_the_new_slots(m, checked):
    say("PA_CHECK decode_step")
    q, kc, vc, bt, cl = decode_case()
    nk, nv = randn(3, 2, 64, seed=8), randn(3, 2, 64, seed=9)
    pos = cl.long() - 1
    slots = torch.where(pos >= 0, bt.long().gather(1, (pos.clamp(min=0) // BS)[:, None])[:, 0] * BS + pos % BS,
                        torch.full_like(pos, -1))
    m.decode_step(nk, nv, slots, torch.empty_like(q), q, kc, vc, bt, cl, 0.125)
    slots[1] = slots[0]
    refused(m, lambda: m.decode_step(nk, nv, slots, torch.empty_like(q), q, kc, vc, bt, cl, 0.125),
            "both write slot")


def prefill_case():
    q_lens, ctx = [3, 5], [10, 5]
    q_, kc, vc, bt, cl = decode_case(ctx=tuple(ctx), HQ=4, HKV=2, D=64)
    q = randn(sum(q_lens), 4, 64, seed=10)
    cu = torch.tensor([0, 3, 8], dtype=torch.int32, device="cuda")
    return q, cu, kc, vc, bt, cl


def test_valid_prefill_runs_as_without_the_check(m, checked):
    say("PA_CHECK valid prefill_attention")
    q, cu, kc, vc, bt, cl = prefill_case()
    a = m.prefill_attention(torch.empty_like(q), q, cu, kc, vc, bt, cl, 0.125)
    checked.delenv("PA_CHECK")
    b = m.prefill_attention(torch.empty_like(q), q, cu, kc, vc, bt, cl, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("case", ["offsets going back", "chunk past its context", "offsets past the tokens"])
def test_bad_prefill_metadata_is_refused(m, checked, case):
    say(f"PA_CHECK prefill_attention: {case}")
    q, cu, kc, vc, bt, cl = prefill_case()
    if case == "offsets going back":
        cu[1], text = 9, "decreases"
    elif case == "chunk past its context":
        cl[0], text = 2, "longer than its context"
    else:  # (sequence 1's context raised so that only the end of the offsets is wrong)
        cu[2], cl[1], text = 9, 9, "past the 8 packed tokens"
    refused(m, lambda: m.prefill_attention(torch.empty_like(q), q, cu, kc, vc, bt, cl, 0.125), text)


def test_mla_decode_checks_its_tables(m, checked):
    say("PA_CHECK mla_decode_attention")
    B, H, QK, R, DC, DV, W = 2, 16, 64, 64, 512, 64, 4
    ctx = (20, 33)
    _, _, _, bt, cl = decode_case(ctx=ctx, W=W)
    cache = randn(NB, BS, DC + R, seed=12)
    qn, qr = randn(B, H, QK, seed=13), randn(B, H, R, seed=14)
    wuk, wuv = randn(DC, H * QK, seed=15) * 0.05, randn(DC, H * DV, seed=16) * 0.05
    out = torch.empty((B, H, DV), dtype=torch.bfloat16, device="cuda")
    m.mla_decode_attention(out, qn, qr, wuk, wuv, cache, bt, cl, 0.1)
    bt[1, 1] = -5
    refused(m, lambda: m.mla_decode_attention(out, qn, qr, wuk, wuv, cache, bt, cl, 0.1), "outside the pool")


def test_mla_decode_step_checks_the_new_slots(m, checked):
    say("PA_CHECK mla_decode_step")
    B, H, QK, R, DC, DV, W = 2, 16, 64, 64, 512, 64, 4
    ctx = (20, 33)
    _, _, _, bt, cl = decode_case(ctx=ctx, W=W)
    cache = randn(NB, BS, DC + R, seed=17)
    qn, qr = randn(B, H, QK, seed=18), randn(B, H, R, seed=19)
    wuk, wuv = randn(DC, H * QK, seed=20) * 0.05, randn(DC, H * DV, seed=21) * 0.05
    nc, nr = randn(B, DC, seed=22), randn(B, R, seed=23)
    out = torch.empty((B, H, DV), dtype=torch.bfloat16, device="cuda")
    pos = cl.long() - 1
    slots = bt.long().gather(1, (pos // BS)[:, None])[:, 0] * BS + pos % BS
    m.mla_decode_step(nc, nr, slots, out, qn, qr, wuk, wuv, cache, bt, cl, 0.1)
    before = cache.clone()
    slots[1] = slots[0]
    refused(m, lambda: m.mla_decode_step(nc, nr, slots, out, qn, qr, wuk, wuv, cache, bt, cl, 0.1),
            "both write slot")
    torch.cuda.synchronize()
    assert torch.equal(cache, before)

