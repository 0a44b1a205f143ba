"""The algorithmic byte counts behind the bench's roofline figures, checked by
walking a small decode workload element by element: every cached position read
once per KV head for K and for V, one block-table entry per block a sequence
touches, its context length, q in and out once per q head, the two scales when
the cache is fp8; and the new-token write of one row per sequence. Likewise the
chunked-prefill flop count, by walking every query row's causal keys."""
import numpy as np
import pytest

import bench
import workloads


def walk_bytes(w):
    e_kv = 1 if w.cache_dtype == "fp8" else 2
    kv = table = 0
    for b in range(w.num_seqs):
        seen_blocks = set()
        for p in range(int(w.context_lens[b])):
            for _h in range(w.num_kv_heads):
                kv += 2 * w.head_size * e_kv  # the position's K row and V row of this head
            seen_blocks.add(int(w.block_tables[b][p // w.block_size]))
        table += 4 * len(seen_blocks)
    lens = 4 * w.num_seqs
    qo = 0
    for _b in range(w.num_seqs):
        for _h in range(w.num_q_heads):
            qo += w.head_size * 2 + w.head_size * 2  # q in (bf16), out (bf16)
    scales = 8 if w.k_scale is not None else 0
    write = 0
    for _b in range(w.num_seqs):
        write += 8  # the token's slot
        for _h in range(w.num_kv_heads):
            write += 2 * w.head_size * (2 + e_kv)  # bf16 K and V in, cache rows out
    return kv, kv + table + lens + qo + scales, write


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [16, 32])
def test_decode_bytes_match_a_walk_of_the_workload(cache, bs):
    rng = np.random.default_rng(7 + bs)
    ctx = rng.integers(1, 200, size=6).astype(np.int32)
    width = int(-(-ctx.max() // bs))
    kw = dict(cache_dtype="fp8", k_scale=0.05, v_scale=0.04) if cache == "fp8" else {}
    w = workloads.make_decode("walk", 99, 6, ctx, rng, num_blocks=int(6 * width + 3), width=width,
                              num_q_heads=4, num_kv_heads=2, head_size=64, block_size=bs, **kw)
    assert bench.decode_bytes(w) == walk_bytes(w)


def walk_prefill_flops(w):
    """Each packed query row is the last positions of its sequence's context; it
    attends causally to every position up to and including its own."""
    D, HQ = w["head_size"], w["num_q_heads"]
    flops = 0
    for b in range(w["num_seqs"]):
        cu0, cu1, L = int(w["cu_seqlens_q"][b]), int(w["cu_seqlens_q"][b + 1]), int(w["context_lens"][b])
        for r in range(cu1 - cu0):
            own = L - (cu1 - cu0) + r  # this row's position
            for _key in range(max(own + 1, 0)):
                flops += HQ * (2 * D + 2 * D)  # q.k and p*v over D, every q head
    return flops


def test_prefill_flops_match_a_walk_of_the_workload():
    w = workloads.prefill_chunks(num_seqs=3, chunk=40, prefix_hi=90, num_blocks=64)
    assert bench.prefill_flops(w) == walk_prefill_flops(w)


def test_bulk_write_bytes_match_a_walk_of_the_workload():
    w = workloads.prefill_write_fp8(num_tokens=300)
    nbytes = 0
    for t in range(w["num_tokens"]):
        nbytes += 8  # the token's slot
        if w["slot_mapping"][t] >= 0:
            for _h in range(w["num_heads"]):
                nbytes += 2 * w["head_size"] * (2 + 1)  # K and V: bf16 row in, fp8 row out
    assert bench.bulk_write_bytes(w) == nbytes


def test_mla_algorithmic_bytes_match_a_walk_of_the_workload():
    """Latent rows (latent + RoPE part, bf16) once per cached position, one table
    entry per block, the lengths, W_UK and W_UV once, q (nope + RoPE) in and the
    output out once per head; the workspace of the design is not counted."""
    w = workloads.mla_decode_b64(num_seqs=3, ctx_lo=5, ctx_hi=70, num_blocks=64, width=8)
    H, QK, R, DC, DV = w["num_heads"], w["qk_nope_dim"], w["rope_dim"], w["kv_lora_rank"], w["v_dim"]
    nbytes = DC * H * QK * 2 + DC * H * DV * 2  # the two up-projections, bf16
    for b in range(w["num_seqs"]):
        blocks = set()
        for p in range(int(w["context_lens"][b])):
            nbytes += (DC + R) * 2
            blocks.add(int(w["block_tables"][b][p // w["block_size"]]))
        nbytes += 4 * len(blocks) + 4
        nbytes += H * ((QK + R) * 2 + DV * 2)
    assert bench.mla_bytes(w)["algorithmic"] == nbytes


def test_mla_segments_match_a_walk_of_the_unit_ranges():
    """Each workgroup of the persistent split owns a contiguous run of the
    units of all sequences (sequence order: a sequence with tiles of 32
    positions gives one unit for its absorbed query, then one per tile; the
    first T % G runs one unit longer); a segment is one sequence whose tiles a
    workgroup sees (a run holding only a query unit makes none)."""
    rng = np.random.default_rng(5)
    for grid in (1, 3, 7, 256):
        ctx = rng.integers(0, 300, size=int(rng.integers(1, 40)))
        units = []  # (sequence, is a tile)
        for b, c in enumerate(ctx):
            n = int(-(-int(c) // 32))
            if n:
                units += [(b, False)] + [(b, True)] * n
        T = len(units)
        segs = 0
        for w in range(grid):
            lo = w * (T // grid) + min(w, T % grid)
            hi = (w + 1) * (T // grid) + min(w + 1, T % grid)
            segs += len({b for b, tile in units[lo:hi] if tile})
        assert bench.mla_segments(ctx, grid) == segs
