"""Pins of the oracle's MLA decode over a latent paged cache (reading R13). CPU only.

Pins:
  * the page's own remark that MLA contains GQA: with a latent that is K and V
    side by side and W_UK / W_UV that only select, MLA decode is the (already
    pinned) GQA decode oracle;
  * library special case: torch scaled_dot_product_attention in fp64 on K and
    V up-projected with torch matmuls, the RoPE part concatenated to q and k;
  * the absorbed form (a different association of the same products): scores
    from (W_UK q) against the latent, values as (P C) W_UV;
  * closed forms: one cached position gives c W_UV exactly; ctx 0 gives zeros;
  * invariants: an out-of-pool table entry removes its positions; relabelling
    physical blocks changes nothing."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits(x):
    return (torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


def make_mla(rng, ctx, H=4, QK=16, R=8, DC=32, DV=16, bs=4, spare=3, w_std=None):
    ctx = np.asarray(ctx, dtype=np.int32)
    nblk = [-(-int(c) // bs) for c in ctx]
    nb = sum(nblk) + spare
    W = max(max(nblk), 1)
    perm = rng.permutation(nb).astype(np.int32)
    bt = workloads.deal_block_tables(perm, ctx, bs, W)
    w_std = w_std or 1.0 / np.sqrt(DC)
    return dict(
        ctx=ctx, bt=bt, bs=bs, H=H, QK=QK, R=R, DC=DC, DV=DV,
        cache=workloads.normal_bf16_bits(rng, (nb, bs, DC + R)),
        q_nope=workloads.normal_bf16_bits(rng, (len(ctx), H, QK)),
        q_rope=workloads.normal_bf16_bits(rng, (len(ctx), H, R)) if R else None,
        w_uk=bf16_bits(rng.normal(0, w_std, (DC, H * QK))),
        w_uv=bf16_bits(rng.normal(0, w_std, (DC, H * DV))))


def run(m, scale, **over):
    a = dict(m, **over)
    return oracle.mla_decode(a["q_nope"], a["q_rope"], a["w_uk"], a["w_uv"], a["cache"], a["bt"],
                             a["ctx"], scale)


def dense_latent(m, b):
    pos = np.arange(int(m["ctx"][b]))
    return f64(m["cache"])[m["bt"][b][pos // m["bs"]], pos % m["bs"]]      # [L, DC + R]


def test_gqa_is_mla_with_selection_matrices():
    """Page: if the latent is large enough to hold K and V and W_UK / W_UV only
    select, MLA implements GQA (with the matching q-group to kv-head relation)."""
    rng = np.random.default_rng(1)
    B, HQ, HKV, D, bs = 3, 8, 2, 16, 4
    ctx = np.array([5, 13, 1], dtype=np.int32)
    nb = 12
    kc = workloads.normal_bf16_bits(rng, (nb, bs, HKV, D))
    vc = workloads.normal_bf16_bits(rng, (nb, bs, HKV, D))
    bt = workloads.deal_block_tables(rng.permutation(nb).astype(np.int32), ctx, bs, 4)
    q = workloads.normal_bf16_bits(rng, (B, HQ, D))
    gqa = oracle.decode_attention(q, oracle.BF16, kc, vc, oracle.BF16, bt, ctx, 0.3)
    DC = 2 * HKV * D
    latent = np.concatenate([kc.reshape(nb, bs, HKV * D), vc.reshape(nb, bs, HKV * D)], axis=2)
    G = HQ // HKV
    wuk = np.zeros((DC, HQ * D), dtype=np.float32)
    wuv = np.zeros((DC, HQ * D), dtype=np.float32)
    for h in range(HQ):
        g = h // G
        for j in range(D):
            wuk[g * D + j, h * D + j] = 1.0
            wuv[HKV * D + g * D + j, h * D + j] = 1.0
    mla = oracle.mla_decode(q, None, bf16_bits(wuk), bf16_bits(wuv), np.ascontiguousarray(latent), bt,
                            ctx, 0.3)
    np.testing.assert_allclose(mla, gqa, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("R", [0, 8])
def test_matches_sdpa_on_up_projected_kv(R):
    rng = np.random.default_rng(2 + R)
    m = make_mla(rng, [7, 1, 22, 16], R=R)
    scale = 0.17
    got = run(m, scale)
    for b in range(len(m["ctx"])):
        C = torch.from_numpy(dense_latent(m, b))
        K = (C[:, :m["DC"]] @ torch.from_numpy(f64(m["w_uk"]))).view(-1, m["H"], m["QK"])
        V = (C[:, :m["DC"]] @ torch.from_numpy(f64(m["w_uv"]))).view(-1, m["H"], m["DV"])
        q = torch.from_numpy(f64(m["q_nope"][b]))                                  # [H, QK]
        if R:
            kr = C[:, m["DC"]:].unsqueeze(1).expand(-1, m["H"], -1)                 # shared by heads
            K = torch.cat([K, kr], dim=2)
            q = torch.cat([q, torch.from_numpy(f64(m["q_rope"][b]))], dim=1)
        o = torch.nn.functional.scaled_dot_product_attention(
            q[:, None, :].contiguous(), K.permute(1, 0, 2).contiguous(), V.permute(1, 0, 2).contiguous(),
            scale=scale)
        np.testing.assert_allclose(got[b], o[:, 0, :].numpy(), rtol=1e-12, atol=1e-12)


def test_absorbed_form_gives_the_same_output():
    rng = np.random.default_rng(4)
    m = make_mla(rng, [9, 30, 3], H=4, QK=16, R=8, DC=32, DV=8)
    got = run(m, 0.2)
    wuk, wuv = f64(m["w_uk"]), f64(m["w_uv"])
    for b in range(3):
        C = dense_latent(m, b)
        for h in range(m["H"]):
            qt = wuk[:, h * 16:(h + 1) * 16] @ f64(m["q_nope"][b, h])               # W_UK,h q_h  [DC]
            s = 0.2 * (C[:, :32] @ qt + C[:, 32:] @ f64(m["q_rope"][b, h]))
            p = np.exp(s - s.max())
            o = (p @ C[:, :32]) / p.sum() @ wuv[:, h * 8:(h + 1) * 8]
            np.testing.assert_allclose(got[b, h], o, rtol=1e-12, atol=1e-12)


def test_one_position_and_empty_context():
    rng = np.random.default_rng(5)
    m = make_mla(rng, [1, 0, 1])
    got = run(m, 0.5)
    assert np.all(got[1] == 0)
    wuv = f64(m["w_uv"])
    for b in (0, 2):
        c = dense_latent(m, b)[0, :m["DC"]]
        ref = (c @ wuv).reshape(m["H"], m["DV"])
        np.testing.assert_allclose(got[b], ref, rtol=1e-14, atol=1e-14)


def test_bad_table_entry_drops_its_positions_and_relabelling_is_exact():
    rng = np.random.default_rng(6)
    m = make_mla(rng, [12, 9], bs=4, spare=6)
    base = run(m, 0.25)
    # relabel physical blocks
    nb = m["cache"].shape[0]
    perm = rng.permutation(nb)
    c2 = np.empty_like(m["cache"])
    c2[perm] = m["cache"]
    bt2 = np.where(m["bt"] >= 0, perm[np.maximum(m["bt"], 0)], -1).astype(np.int32)
    assert np.array_equal(run(m, 0.25, cache=c2, bt=bt2), base)
    # sequence 0's middle block outside the pool == that sequence without those 4 positions
    bad = m["bt"].copy()
    bad[0, 1] = nb + 5
    got = run(m, 0.25, bt=bad)
    keep = [0, 1, 2, 3, 8, 9, 10, 11]
    C = dense_latent(m, 0)[keep]
    wuk, wuv = f64(m["w_uk"]), f64(m["w_uv"])
    for h in range(m["H"]):
        k = C[:, :m["DC"]] @ wuk[:, h * 16:(h + 1) * 16]
        s = 0.25 * (k @ f64(m["q_nope"][0, h]) + C[:, m["DC"]:] @ f64(m["q_rope"][0, h]))
        p = np.exp(s - s.max())
        o = p @ (C[:, :m["DC"]] @ wuv[:, h * 16:(h + 1) * 16]) / p.sum()
        np.testing.assert_allclose(got[0, h], o, rtol=1e-12, atol=1e-12)
    assert np.array_equal(got[1], base[1])
