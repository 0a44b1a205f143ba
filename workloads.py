"""Seeded synthetic inputs shaped like the Qwen3-0.6B paged-KV workloads.

This module only draws inputs: random values, permutations, context lengths,
block tables and slot mappings (the engine's bookkeeping that places token p of
sequence b in block ``table[b][p // bs]`` at offset ``p % bs``). It holds none of
the kernels' arithmetic, and both the CPU oracle and the GPU path take their
inputs from here, so both sides always see the same bytes.

Recipe (every workload is seeded by ``numpy.random.PCG64(SeedSequence([304, id]))``):
  - float tensors are drawn as fp32 standard normals (times a stated standard
    deviation) and rounded to bf16 by torch's round-to-nearest-even cast;
  - fp8 e4m3fn caches hold what the scaled cache write makes of N(0,1) data:
    fp32 normals rounded to bf16, divided by the per-tensor scale in fp32 and
    cast to e4m3fn (round to nearest even) by torch;
  - large pools are drawn on the target device with a torch Generator seeded
    from the same SeedSequence (bit-identical between runs on one device);
  - physical blocks are handed out in the order of a seeded permutation of the
    pool, ceil(ctx/bs) blocks per sequence; unused table entries are -1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

SEED_ROOT = 304


def rng_for(workload_id: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, workload_id,
                                                                       *extra])))


def torch_seed(rng: np.random.Generator) -> int:
    return int(rng.integers(0, 2**62))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with torch's cast; return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_bf16_bits(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return bf16_bits_from_f32(x)


def normal_fp8_codes(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    """fp8 cache contents as the scaled cache write makes them from N(0,1) data:
    fp32 normals rounded to bf16, divided by the fp32 scale (numpy's IEEE fp32
    division), cast to e4m3fn by torch (round to nearest even)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    y = xb / np.float32(scale)
    return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def device_fp8(shape, device, seed: int, scale: float, chunk_elems: int = 1 << 28) -> torch.Tensor:
    """Seeded fp8 e4m3fn cache drawn on ``device`` by the recipe of
    ``normal_fp8_codes``: N(0,1) -> bf16 -> / scale (fp32) -> e4m3fn, by torch ops."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.float8_e4m3fn, device=device)
    flat = out.view(-1)
    sc = torch.tensor(float(np.float32(scale)), dtype=torch.float32, device=device)
    n = flat.numel()
    for start in range(0, n, chunk_elems):
        m = min(chunk_elems, n - start)
        x = torch.randn(m, generator=g, device=device, dtype=torch.float32)
        x = x.to(torch.bfloat16).float().div_(sc)
        flat[start:start + m].copy_(x.to(torch.float8_e4m3fn))
        del x
    return out


def device_normal(shape, dtype: torch.dtype, device, seed: int, std: float = 1.0,
                  chunk_elems: int = 1 << 28) -> torch.Tensor:
    """Seeded normal tensor drawn on ``device`` (chunked to bound scratch memory):
    N(0, std^2) in fp32, rounded to ``dtype`` by torch's cast (fp8 caches of the
    workloads come from ``device_fp8``)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for start in range(0, n, chunk_elems):
        m = min(chunk_elems, n - start)
        x = torch.randn(m, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[start:start + m].copy_(x.to(dtype))
        del x
    return out


# --------------------------------------------------------------------------- #
# Paged layouts
# --------------------------------------------------------------------------- #

def deal_block_tables(perm: np.ndarray, context_lens: np.ndarray, block_size: int,
                      width: int) -> np.ndarray:
    """Give sequence b the next ceil(ctx_b/bs) blocks of ``perm``; pad with -1."""
    B = context_lens.shape[0]
    bt = np.full((B, width), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        nblk = -(-int(context_lens[b]) // block_size)
        assert nblk <= width and pos + nblk <= perm.shape[0]
        bt[b, :nblk] = perm[pos:pos + nblk]
        pos += nblk
    return bt


def slots_for_positions(block_tables: np.ndarray, seq_ids: np.ndarray, positions: np.ndarray,
                        block_size: int) -> np.ndarray:
    """Slot that the engine assigns to position p of sequence b (block-manager bookkeeping)."""
    blk = block_tables[seq_ids, positions // block_size].astype(np.int64)
    return blk * block_size + (positions % block_size)


@dataclass
class DecodeWorkload:
    """Metadata of one decode step over a paged pool (tensors are drawn separately)."""
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray          # int32 [B, W]
    new_token_slots: np.ndarray       # int64 [B]: slot of position ctx_b - 1
    softmax_scale: float
    cache_dtype: str                  # "bf16" | "fp8"
    k_scale: Optional[float] = None
    v_scale: Optional[float] = None
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def width(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_read_bytes(self) -> int:
        esz = 1 if self.cache_dtype == "fp8" else 2
        return int(2 * int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads
                   * self.head_size * esz)


def make_decode(name: str, workload_id: int, num_seqs: int, context_lens: np.ndarray,
                rng: np.random.Generator, num_blocks: int, width: int, num_q_heads: int = 16,
                num_kv_heads: int = 8, head_size: int = 128, block_size: int = 16,
                cache_dtype: str = "bf16", k_scale=None, v_scale=None) -> DecodeWorkload:
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = deal_block_tables(perm, context_lens, block_size, width)
    seq = np.arange(num_seqs)
    new_slots = slots_for_positions(bt, seq, context_lens.astype(np.int64) - 1, block_size)
    return DecodeWorkload(name=name, num_seqs=num_seqs, num_q_heads=num_q_heads,
                          num_kv_heads=num_kv_heads, head_size=head_size, block_size=block_size,
                          num_blocks=num_blocks, context_lens=context_lens.astype(np.int32),
                          block_tables=bt, new_token_slots=new_slots,
                          softmax_scale=float(np.float32(1.0 / math.sqrt(head_size))),
                          cache_dtype=cache_dtype, k_scale=k_scale, v_scale=v_scale,
                          seed=torch_seed(rng))


def qwen3_decode_b64(num_seqs: int = 64, ctx_lo: int = 512, ctx_hi: int = 4096,
                     num_blocks: int = 32768, width: int = 256, workload_id: int = 2,
                     **kw) -> DecodeWorkload:
    """Qwen3-0.6B-shaped single-layer decode, batch 64, ctx ~ U{512..4096}, bf16 cache."""
    rng = rng_for(workload_id)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=num_seqs).astype(np.int32)
    return make_decode("qwen3_0.6b_decode_b64_bf16", workload_id, num_seqs, ctx, rng,
                       num_blocks, width, **kw)


def mixed_decode_fp8(num_seqs: int = 256, median: float = 1024.0, sigma: float = 1.0,
                     cap: int = 8192, num_blocks: int = 65536, width: int = 512,
                     workload_id: int = 4, k_scale: float = 0.05, v_scale: float = 0.04,
                     **kw) -> DecodeWorkload:
    """Batch-256 decode, ctx lognormal (median 1024, sigma 1, capped at 8192), fp8 cache."""
    rng = rng_for(workload_id)
    z = rng.standard_normal(num_seqs)
    ctx = np.clip(np.rint(median * np.exp(sigma * z)), 1, cap).astype(np.int32)
    return make_decode("qwen3_0.6b_decode_b256_fp8_mixed", workload_id, num_seqs, ctx, rng,
                       num_blocks, width, cache_dtype="fp8",
                       k_scale=float(np.float32(k_scale)), v_scale=float(np.float32(v_scale)),
                       **kw)


def tiny_paged(workload_id: int = 1) -> dict:
    """Two sequences (ctx 37 and 64) written token by token into a 16-block pool.

    Returns host arrays: ``slot_mapping`` [101], ``key``/``value`` bf16 bits
    [101, 8, 128], ``q`` bf16 bits [2, 16, 128], ``block_tables`` [2, 4],
    ``context_lens`` [2], plus sizes.
    """
    rng = rng_for(workload_id)
    ctx = np.array([37, 64], dtype=np.int32)
    bs, nb, hkv, hq, d = 16, 16, 8, 16, 128
    perm = rng.permutation(nb).astype(np.int32)
    bt = deal_block_tables(perm, ctx, bs, 4)
    seq = np.concatenate([np.full(int(c), b) for b, c in enumerate(ctx)])
    pos = np.concatenate([np.arange(int(c)) for c in ctx])
    slots = slots_for_positions(bt, seq, pos, bs)
    key = normal_bf16_bits(rng, (seq.shape[0], hkv, d))
    value = normal_bf16_bits(rng, (seq.shape[0], hkv, d))
    q = normal_bf16_bits(rng, (2, hq, d))
    return dict(context_lens=ctx, block_tables=bt, slot_mapping=slots, key=key, value=value, q=q,
                num_blocks=nb, block_size=bs, num_kv_heads=hkv, num_q_heads=hq, head_size=d,
                softmax_scale=float(np.float32(1.0 / math.sqrt(d))))


def prefill_write_fp8(num_tokens: int = 32768, skip_frac: float = 0.05, workload_id: int = 3,
                      num_heads: int = 8, head_size: int = 128, block_size: int = 16) -> dict:
    """Bulk prefill write: permuted slots with 5% skipped, 2*N(0,1) bf16 -> fp8 (0.05/0.04)."""
    rng = rng_for(workload_id)
    slots = rng.permutation(num_tokens).astype(np.int64)
    nskip = int(round(skip_frac * num_tokens))
    skipped = rng.choice(num_tokens, size=nskip, replace=False)
    slots[skipped] = -1
    return dict(slot_mapping=slots, num_tokens=num_tokens, num_heads=num_heads,
                head_size=head_size, block_size=block_size,
                num_blocks=-(-num_tokens // block_size), std=2.0,
                k_scale=float(np.float32(0.05)), v_scale=float(np.float32(0.04)),
                seed=torch_seed(rng))


def mla_concat_swa(num_tokens: int = 16384, num_heads: int = 128, nope_dim: int = 128,
                   rope_dim: int = 64, skip_frac: float = 0.10, block_size: int = 16,
                   workload_id: int = 5) -> dict:
    """MLA-style K assembly then an SWA-remapped K-only bf16 write.

    slot_mapping is a permutation of the slots (no -1); the SWA table is a
    second permutation with 10% of its entries set to -1.
    """
    rng = rng_for(workload_id)
    slots = rng.permutation(num_tokens).astype(np.int64)
    swa = rng.permutation(num_tokens).astype(np.int64)
    nskip = int(round(skip_frac * num_tokens))
    swa[rng.choice(num_tokens, size=nskip, replace=False)] = -1
    return dict(slot_mapping=slots, swa_slot_mapping=swa, num_tokens=num_tokens,
                num_heads=num_heads, nope_dim=nope_dim, rope_dim=rope_dim,
                block_size=block_size, num_blocks=-(-num_tokens // block_size),
                seed=torch_seed(rng))


def prefill_chunks(num_seqs: int = 16, chunk: int = 512, prefix_hi: int = 3584,
                   workload_id: int = 6, num_q_heads: int = 16, num_kv_heads: int = 8,
                   head_size: int = 128, block_size: int = 16, num_blocks: int = 4096) -> dict:
    """Chunked prefill, Qwen3-0.6B heads: 16 sequences each appending a 512-token
    chunk to a cached prefix of U{0..3584} tokens (context = prefix + chunk); the
    chunk's K/V are already in the bf16 pool (4,096 blocks); packed queries with
    cu_seqlens_q. Caches and q are drawn on the device from the returned seed."""
    rng = rng_for(workload_id)
    prefix = rng.integers(0, prefix_hi + 1, size=num_seqs)
    ctx = (prefix + chunk).astype(np.int32)
    nblk = -(-ctx // block_size)
    width = int(-(-(prefix_hi + chunk) // block_size))
    perm = rng.permutation(num_blocks).astype(np.int32)
    assert int(nblk.sum()) <= num_blocks
    bt = deal_block_tables(perm, ctx, block_size, width)
    cu = np.arange(num_seqs + 1, dtype=np.int32) * chunk
    return dict(name=f"prefill_chunks_{num_seqs}x{chunk}_bf16", num_seqs=num_seqs,
                num_tokens=num_seqs * chunk, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                head_size=head_size, block_size=block_size, num_blocks=num_blocks,
                context_lens=ctx, block_tables=bt, cu_seqlens_q=cu,
                softmax_scale=float(np.float32(1.0 / np.sqrt(head_size))),
                seed=torch_seed(rng))


def mla_decode_b64(num_seqs: int = 64, ctx_lo: int = 512, ctx_hi: int = 4096,
                   num_blocks: int = 32768, width: int = 256, workload_id: int = 7) -> dict:
    """MLA decode over a latent paged cache, DeepSeek-V2-Lite-shaped (synthetic):
    16 heads, qk_nope 128, RoPE 64, kv_lora_rank 512, v 128, block_size 16, batch 64
    with ctx ~ U{512..4096} (the GQA decode workload's length mix). Weights are
    N(0, 1/512) so that up-projected keys and values have unit scale."""
    rng = rng_for(workload_id)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=num_seqs).astype(np.int32)
    bs = 16
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = deal_block_tables(perm, ctx, bs, width)
    H, QK, R, DC, DV = 16, 128, 64, 512, 128
    new_slots = slots_for_positions(bt, np.arange(num_seqs), ctx.astype(np.int64) - 1, bs)
    return dict(name="mla_latent_decode_b64", num_seqs=num_seqs, num_heads=H, qk_nope_dim=QK,
                rope_dim=R, kv_lora_rank=DC, v_dim=DV, block_size=bs, num_blocks=num_blocks,
                context_lens=ctx, block_tables=bt, new_token_slots=new_slots,
                softmax_scale=float(np.float32(1.0 / math.sqrt(QK + R))), w_std=1.0 / math.sqrt(DC),
                seed=torch_seed(rng))
