"""torch-tensor front ends of the C entry points (argument marshalling only).

Each function checks what a tensor can tell (device, dtype, rank, strides),
passes raw device pointers, element strides and the current HIP stream to the
library, and raises ``PagedKVError`` on a non-OK status. All arithmetic happens
in the HIP kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import PA_BF16, PA_F32, PA_FP8_E4M3FN, check, lib

_DTYPES = {torch.bfloat16: PA_BF16, torch.float32: PA_F32, torch.float8_e4m3fn: PA_FP8_E4M3FN}


def _code(t: torch.Tensor, what: str) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise _lib.PagedKVError(_lib.PA_EDTYPE, f"{what}: unsupported dtype {t.dtype}") from None


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _on_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("pagedkv: every tensor must live on the GPU")


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _scratch(nbytes: int, device, stream=None) -> torch.Tensor:
    """Workspace allocated on the stream the kernels run on: the caching allocator
    then hands its memory out again only in that stream's order, i.e. after them."""
    s = stream if stream is not None else torch.cuda.current_stream(device)
    with torch.cuda.stream(s):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def reshape_and_cache(key: torch.Tensor, value: Optional[torch.Tensor], key_cache: torch.Tensor,
                      value_cache: Optional[torch.Tensor], slot_mapping: torch.Tensor,
                      swa_slot_mapping: Optional[torch.Tensor] = None,
                      k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """Write ``key``/``value`` [T, H, D] into ``key_cache``/``value_cache`` [NB, BS, H, D]."""
    _on_gpu(key, value, key_cache, value_cache, slot_mapping, swa_slot_mapping, k_scale, v_scale)
    if key.dim() != 3 or key_cache.dim() != 4:
        raise ValueError("key must be [T, H, D] and key_cache [NB, BS, H, D]")
    T, H, D = key.shape
    NB, BS, H2, D2 = key_cache.shape
    if (H2, D2) != (H, D):
        raise ValueError(f"cache heads/dims {(H2, D2)} differ from source {(H, D)}")
    if key.stride(2) != 1 or key.stride(1) != D:
        raise ValueError("key must have head stride D and unit dim stride")
    if key_cache.stride(3) != 1 or key_cache.stride(2) != D or key_cache.stride(1) != H * D:
        raise ValueError("key_cache inner [BS, H, D] must be contiguous")
    if value is not None:
        if value.shape != key.shape or value.stride(2) != 1 or value.stride(1) != D:
            raise ValueError("value must match key")
        if value_cache is None or value_cache.shape != key_cache.shape or \
                value_cache.stride() != key_cache.stride() or value_cache.dtype != key_cache.dtype:
            raise ValueError("value_cache must match key_cache")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != T or \
            not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous int64 [T]")
    if swa_slot_mapping is not None and (swa_slot_mapping.dtype != torch.int64
                                         or not swa_slot_mapping.is_contiguous()):
        raise ValueError("swa_slot_mapping must be contiguous int64")
    for s in (k_scale, v_scale):
        if s is not None and (s.dtype != torch.float32 or s.numel() != 1):
            raise ValueError("scales must be single fp32 device scalars")
    check(lib.pa_reshape_and_cache(
        key.data_ptr(), _ptr(value), _code(key, "key"), T, H, D, key.stride(0),
        value.stride(0) if value is not None else 0, key_cache.data_ptr(), _ptr(value_cache),
        _code(key_cache, "key_cache"), NB, BS, key_cache.stride(0),
        slot_mapping.data_ptr(), _ptr(swa_slot_mapping),
        swa_slot_mapping.numel() if swa_slot_mapping is not None else 0,
        _ptr(k_scale), _ptr(v_scale), _stream(stream)))


def concat_and_cast_mla_k(k: torch.Tensor, k_nope: torch.Tensor, k_rope: torch.Tensor,
                          stream=None) -> None:
    """``k[t, h, :] = cast(k_nope[t, h, :] ++ k_rope[t, 0, :])`` in place."""
    _on_gpu(k, k_nope, k_rope)
    if k.dim() != 3 or k_nope.dim() != 3 or k_rope.dim() != 3:
        raise ValueError("k, k_nope and k_rope must be 3-D")
    T, H, KD = k.shape
    if k_nope.shape[0] != T or k_rope.shape[0] != T:
        raise ValueError("token counts differ")
    if k_nope.shape[1] != H or k_rope.shape[1] != 1:
        raise ValueError("k_nope must have k's heads and k_rope a single head")
    nope, rope = k_nope.shape[2], k_rope.shape[2]
    if KD != nope + rope:
        raise ValueError("k's last dim must equal nope_dim + rope_dim")
    for t in (k, k_nope, k_rope):
        if t.numel() > 0 and t.stride(2) != 1:
            raise ValueError("innermost strides must be 1")
    check(lib.pa_concat_and_cast_mla_k(
        k.data_ptr(), _code(k, "k"), k.stride(0), k.stride(1), k_nope.data_ptr(),
        _code(k_nope, "k_nope"), k_nope.stride(0), k_nope.stride(1), k_rope.data_ptr(),
        _code(k_rope, "k_rope"), k_rope.stride(0), T, H, nope, rope, _stream(stream)))


def concat_and_cache_mla_k(k_nope: torch.Tensor, k_rope: torch.Tensor, key_cache: torch.Tensor,
                           slot_mapping: torch.Tensor,
                           swa_slot_mapping: Optional[torch.Tensor] = None,
                           k_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """k_nope [T, H, nope] ++ k_rope [T, 1, rope], cast and written straight into
    ``key_cache`` [NB, BS, H, nope + rope] through the slot mapping (optional SWA
    table and k_scale as in reshape_and_cache)."""
    _on_gpu(k_nope, k_rope, key_cache, slot_mapping, swa_slot_mapping, k_scale)
    T, H, nope = k_nope.shape
    rope = k_rope.shape[2]
    NB, BS, H2, kd = key_cache.shape
    if k_rope.shape[:2] != (T, 1) or H2 != H or kd != nope + rope:
        raise ValueError("k_nope [T, H, nope], k_rope [T, 1, rope], key_cache [NB, BS, H, nope + rope]")
    if k_nope.dtype != k_rope.dtype:
        raise ValueError("k_nope and k_rope dtypes differ")
    if k_nope.stride(2) != 1 or (rope > 0 and k_rope.stride(2) != 1):
        raise ValueError("source rows must be contiguous")
    if key_cache.stride(3) != 1 or key_cache.stride(2) != kd or key_cache.stride(1) != H * kd:
        raise ValueError("cache inner [BS, H, nope + rope] must be contiguous")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous() or slot_mapping.numel() != T:
        raise ValueError("slot_mapping must be contiguous int64 [T]")
    swa_len = 0
    if swa_slot_mapping is not None:
        if swa_slot_mapping.dtype != torch.int64 or not swa_slot_mapping.is_contiguous():
            raise ValueError("swa_slot_mapping must be contiguous int64")
        swa_len = swa_slot_mapping.numel()
    check(lib.pa_concat_and_cache_mla_k(
        k_nope.data_ptr(), _code(k_nope, "k_nope"), k_nope.stride(0), k_nope.stride(1),
        k_rope.data_ptr(), k_rope.stride(0), T, H, nope, rope, key_cache.data_ptr(),
        _code(key_cache, "key_cache"), NB, BS, key_cache.stride(0), slot_mapping.data_ptr(),
        _ptr(swa_slot_mapping), swa_len, _ptr(k_scale), _stream(stream)))


def decode_attention_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                    head_size: int, max_blocks_per_seq: int,
                                    block_size: int) -> int:
    n = int(lib.pa_decode_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_size,
                                                   max_blocks_per_seq, block_size))
    if n == 0:
        raise _lib.PagedKVError(_lib.PA_EINVAL, _lib.last_error())
    return n


def decode_attention(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                     value_cache: torch.Tensor, block_tables: torch.Tensor,
                     context_lens: torch.Tensor, softmax_scale: float,
                     k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Single-token paged decode attention; writes and returns ``out`` [B, H_Q, D]."""
    _on_gpu(out, q, key_cache, value_cache, block_tables, context_lens, k_scale, v_scale, workspace)
    B, HQ, D = q.shape
    NB, BS, HKV, D2 = key_cache.shape
    if D2 != D or out.shape != q.shape:
        raise ValueError("q, out and cache head sizes differ")
    if q.stride(2) != 1 or q.stride(1) != D or out.stride(2) != 1 or out.stride(1) != D:
        raise ValueError("q and out must be [B, H_Q, D] with contiguous [H_Q, D]")
    if key_cache.stride(3) != 1 or key_cache.stride(2) != D or key_cache.stride(1) != HKV * D:
        raise ValueError("cache inner [BS, H_KV, D] must be contiguous")
    if value_cache.shape != key_cache.shape or value_cache.stride() != key_cache.stride() or \
            value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != B or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [B, W]")
    if context_lens.dtype != torch.int32 or context_lens.numel() != B or \
            not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    W = block_tables.shape[1]
    need = decode_attention_workspace_size(max(B, 1), HQ, HKV, D, W, BS)
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    check(lib.pa_decode_attention(
        out.data_ptr(), _code(out, "out"), out.stride(0), q.data_ptr(), _code(q, "q"), q.stride(0),
        key_cache.data_ptr(), value_cache.data_ptr(), _code(key_cache, "key_cache"), NB, BS,
        key_cache.stride(0), block_tables.data_ptr(), W, context_lens.data_ptr(), B, HQ, HKV, D,
        float(softmax_scale), _ptr(k_scale), _ptr(v_scale), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def decode_attention_noalloc(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                             value_cache: torch.Tensor, block_tables: torch.Tensor,
                             context_lens: torch.Tensor, softmax_scale: float,
                             k_scale: Optional[torch.Tensor] = None,
                             v_scale: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``decode_attention`` with the library's fixed device workspace: neither this
    function nor the C call allocates. Calls that overlap on one GPU race."""
    _on_gpu(out, q, key_cache, value_cache, block_tables, context_lens, k_scale, v_scale)
    B, HQ, D = q.shape
    NB, BS, HKV, D2 = key_cache.shape
    if D2 != D or out.shape != q.shape:
        raise ValueError("q, out and cache head sizes differ")
    if q.stride(2) != 1 or q.stride(1) != D or out.stride(2) != 1 or out.stride(1) != D:
        raise ValueError("q and out must be [B, H_Q, D] with contiguous [H_Q, D]")
    if key_cache.stride(3) != 1 or key_cache.stride(2) != D or key_cache.stride(1) != HKV * D:
        raise ValueError("cache inner [BS, H_KV, D] must be contiguous")
    if value_cache.shape != key_cache.shape or value_cache.stride() != key_cache.stride() or \
            value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != B or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [B, W]")
    if context_lens.dtype != torch.int32 or context_lens.numel() != B or \
            not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    check(lib.pa_decode_attention_noalloc(
        out.data_ptr(), _code(out, "out"), out.stride(0), q.data_ptr(), _code(q, "q"), q.stride(0),
        key_cache.data_ptr(), value_cache.data_ptr(), _code(key_cache, "key_cache"), NB, BS,
        key_cache.stride(0), block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(),
        B, HQ, HKV, D, float(softmax_scale), _ptr(k_scale), _ptr(v_scale), _stream(stream)))
    return out


def decode_step(new_k: torch.Tensor, new_v: torch.Tensor, new_slots: torch.Tensor,
                out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                softmax_scale: float, k_scale: Optional[torch.Tensor] = None,
                v_scale: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """One decode step: write each sequence's new token K/V [B, H_KV, D] (bf16)
    into its slot, then single-token decode attention; writes and returns ``out``."""
    _on_gpu(new_k, new_v, new_slots, out, q, key_cache, value_cache, block_tables, context_lens,
            k_scale, v_scale, workspace)
    B, HQ, D = q.shape
    NB, BS, HKV, D2 = key_cache.shape
    if new_k.shape != (B, HKV, D) or new_v.shape != (B, HKV, D):
        raise ValueError("new_k / new_v must be [B, H_KV, D]")
    if new_k.stride(2) != 1 or new_k.stride(1) != D or new_v.stride(2) != 1 or new_v.stride(1) != D:
        raise ValueError("new_k / new_v rows must be contiguous [H_KV, D]")
    if new_slots.dtype != torch.int64 or new_slots.numel() != B or not new_slots.is_contiguous():
        raise ValueError("new_slots must be contiguous int64 [B]")
    if D2 != D or out.shape != q.shape:
        raise ValueError("q, out and cache head sizes differ")
    if q.stride(2) != 1 or q.stride(1) != D or out.stride(2) != 1 or out.stride(1) != D:
        raise ValueError("q and out must be [B, H_Q, D] with contiguous [H_Q, D]")
    if key_cache.stride(3) != 1 or key_cache.stride(2) != D or key_cache.stride(1) != HKV * D:
        raise ValueError("cache inner [BS, H_KV, D] must be contiguous")
    if value_cache.shape != key_cache.shape or value_cache.stride() != key_cache.stride() or \
            value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != B or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [B, W]")
    if context_lens.dtype != torch.int32 or context_lens.numel() != B or \
            not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    W = block_tables.shape[1]
    need = decode_attention_workspace_size(max(B, 1), HQ, HKV, D, W, BS)
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    if new_v.dtype != new_k.dtype:
        raise ValueError("new_k and new_v dtypes differ")
    check(lib.pa_decode_step(
        new_k.data_ptr(), new_v.data_ptr(), _code(new_k, "new_k"), new_k.stride(0), new_v.stride(0),
        new_slots.data_ptr(), out.data_ptr(), _code(out, "out"), out.stride(0), q.data_ptr(),
        _code(q, "q"), q.stride(0), key_cache.data_ptr(), value_cache.data_ptr(),
        _code(key_cache, "key_cache"), NB, BS, key_cache.stride(0), block_tables.data_ptr(), W,
        context_lens.data_ptr(), B, HQ, HKV, D, float(softmax_scale), _ptr(k_scale), _ptr(v_scale),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def prefill_attention(out: torch.Tensor, q: torch.Tensor, cu_seqlens_q: torch.Tensor,
                      key_cache: torch.Tensor, value_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, softmax_scale: float,
                      k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Chunked-prefill paged attention of packed queries ``q`` [T, H_Q, D] (rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 belong to sequence b and are the last
    positions of its context); writes and returns ``out`` [T, H_Q, D]."""
    _on_gpu(out, q, cu_seqlens_q, key_cache, value_cache, block_tables, context_lens, k_scale,
            v_scale)
    T, HQ, D = q.shape
    NB, BS, HKV, D2 = key_cache.shape
    B = context_lens.numel()
    if D2 != D or out.shape != q.shape:
        raise ValueError("q, out and cache head sizes differ")
    if q.stride(2) != 1 or q.stride(1) != D or out.stride(2) != 1 or out.stride(1) != D:
        raise ValueError("q and out must be [T, H_Q, D] with contiguous [H_Q, D]")
    if key_cache.stride(3) != 1 or key_cache.stride(2) != D or key_cache.stride(1) != HKV * D:
        raise ValueError("cache inner [BS, H_KV, D] must be contiguous")
    if value_cache.shape != key_cache.shape or value_cache.stride() != key_cache.stride() or \
            value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_q.numel() != B + 1 or \
            not cu_seqlens_q.is_contiguous():
        raise ValueError("cu_seqlens_q must be contiguous int32 [B + 1]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != B or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [B, W]")
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    check(lib.pa_prefill_attention(
        out.data_ptr(), _code(out, "out"), out.stride(0), q.data_ptr(), _code(q, "q"), q.stride(0), T,
        cu_seqlens_q.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        _code(key_cache, "key_cache"), NB, BS, key_cache.stride(0), block_tables.data_ptr(),
        block_tables.shape[1], context_lens.data_ptr(), B, HQ, HKV, D, float(softmax_scale),
        _ptr(k_scale), _ptr(v_scale), _stream(stream)))
    return out


def hbm_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    """Streaming copy of ``src``'s bytes into ``dst`` (bandwidth reference kernel)."""
    _on_gpu(dst, src)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("dst must be contiguous and at least as large as src")
    check(lib.pa_hbm_copy(dst.data_ptr(), src.data_ptr(), n, _stream(stream)))


HBM_READ_SINK_UNITS = 2048  # PA_HBM_READ_SINK_UNITS


def hbm_read(src: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Streaming read of ``src``'s bytes (read-bandwidth reference kernel). Returns
    ``sink`` (int32 [2048, 4], allocated if not given): partial XOR folds of src's
    16-byte units, whose XOR over the first axis is the XOR of all of them."""
    _on_gpu(src, sink)
    n = src.numel() * src.element_size()
    if not src.is_contiguous() or n % 16 != 0:
        raise ValueError("src must be contiguous with a multiple of 16 bytes")
    if sink is None:
        sink = _scratch(16 * HBM_READ_SINK_UNITS, src.device, stream).view(torch.int32).view(
            HBM_READ_SINK_UNITS, 4)
    elif sink.dtype != torch.int32 or sink.numel() != 4 * HBM_READ_SINK_UNITS or not sink.is_contiguous():
        raise ValueError("sink must be contiguous int32 [2048, 4]")
    check(lib.pa_hbm_read(src.data_ptr(), n, sink.data_ptr(), _stream(stream)))
    return sink


def mla_decode_workspace_size(num_seqs: int, num_heads: int, qk_nope_dim: int, rope_dim: int,
                              kv_lora_rank: int, v_dim: int, max_blocks_per_seq: int,
                              block_size: int) -> int:
    n = int(lib.pa_mla_decode_workspace_size(num_seqs, num_heads, qk_nope_dim, rope_dim, kv_lora_rank,
                                             v_dim, max_blocks_per_seq, block_size))
    if n == 0:
        raise _lib.PagedKVError(_lib.PA_EUNSUPPORTED, _lib.last_error())
    return n


def _mla_args(out, q_nope, q_rope, w_uk, w_uv, latent_cache, block_tables, context_lens, softmax_scale,
              workspace, stream):
    """Checked argument list of pa_mla_decode_attention (shared by the step)."""
    _on_gpu(out, q_nope, q_rope, w_uk, w_uv, latent_cache, block_tables, context_lens, workspace)
    B, H, QK = q_nope.shape
    NB, BS, ROW = latent_cache.shape
    R = 0 if q_rope is None else q_rope.shape[2]
    DC = ROW - R
    if w_uk.shape != (DC, H * QK) or w_uv.dim() != 2 or w_uv.shape[0] != DC or w_uv.shape[1] % H:
        raise ValueError("w_uk must be [kv_lora_rank, H*qk] and w_uv [kv_lora_rank, H*dv]")
    DV = w_uv.shape[1] // H
    if not (w_uk.is_contiguous() and w_uv.is_contiguous()):
        raise ValueError("w_uk and w_uv must be contiguous")
    if out.shape != (B, H, DV) or out.stride(2) != 1 or out.stride(1) != DV:
        raise ValueError("out must be [B, H, dv] with contiguous [H, dv] rows")
    if q_nope.stride(2) != 1 or q_nope.stride(1) != QK:
        raise ValueError("q_nope rows [H, qk] must be contiguous")
    if q_rope is not None and (q_rope.shape[:2] != (B, H) or q_rope.stride(2) != 1 or q_rope.stride(1) != R):
        raise ValueError("q_rope must be [B, H, r] with contiguous [H, r] rows")
    if latent_cache.stride(2) != 1 or latent_cache.stride(1) != ROW:
        raise ValueError("latent_cache inner [BS, row] must be contiguous")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != B or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [B, W]")
    if context_lens.dtype != torch.int32 or context_lens.numel() != B or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    W = block_tables.shape[1]
    if workspace is None:
        workspace = _scratch(mla_decode_workspace_size(max(B, 1), H, QK, R, DC, DV, W, BS),
                             q_nope.device, stream)
    return (out.data_ptr(), _code(out, "out"), out.stride(0), q_nope.data_ptr(), q_nope.stride(0),
            _ptr(q_rope), q_rope.stride(0) if q_rope is not None else 0, _code(q_nope, "q_nope"),
            w_uk.data_ptr(), w_uv.data_ptr(), _code(w_uk, "w_uk"), latent_cache.data_ptr(),
            _code(latent_cache, "latent_cache"), NB, BS, latent_cache.stride(0), block_tables.data_ptr(), W,
            context_lens.data_ptr(), B, H, QK, R, DC, DV, float(softmax_scale), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream(stream))


def mla_decode_attention(out: torch.Tensor, q_nope: torch.Tensor, q_rope: Optional[torch.Tensor],
                         w_uk: torch.Tensor, w_uv: torch.Tensor, latent_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor, softmax_scale: float,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """MLA decode over a paged latent cache [NB, BS, kv_lora_rank + rope_dim]:
    q_nope [B, H, qk], q_rope [B, H, r] (or None), w_uk [kv_lora_rank, H*qk],
    w_uv [kv_lora_rank, H*dv]; writes and returns out [B, H, dv]."""
    check(lib.pa_mla_decode_attention(*_mla_args(out, q_nope, q_rope, w_uk, w_uv, latent_cache, block_tables,
                                                 context_lens, softmax_scale, workspace, stream)))
    return out


def mla_decode_step(new_c: torch.Tensor, new_rope: Optional[torch.Tensor], new_slots: torch.Tensor,
                    out: torch.Tensor, q_nope: torch.Tensor, q_rope: Optional[torch.Tensor],
                    w_uk: torch.Tensor, w_uv: torch.Tensor, latent_cache: torch.Tensor,
                    block_tables: torch.Tensor, context_lens: torch.Tensor, softmax_scale: float,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One MLA decode step: sequence b's new latent row new_c[b] [kv_lora_rank]
    ++ new_rope[b] [rope_dim] (bf16, rows of the trailing dims may be [B, 1, n])
    into latent_cache slot new_slots[b] (int64; negative skips), then
    mla_decode_attention over the cache; returns out."""
    _on_gpu(new_c, new_rope, new_slots)
    B = q_nope.shape[0]
    R = 0 if q_rope is None else q_rope.shape[2]
    DC = latent_cache.shape[2] - R
    def rows(t):  # [B, 1, n] -> the [B, n] view (never a copy: the pointer goes to the launch)
        if t is None or t.dim() != 3:
            return t
        if t.shape[1] != 1:
            raise ValueError("new rows must be [B, n] or [B, 1, n]")
        return t[:, 0, :]
    c2, r2 = rows(new_c), rows(new_rope)
    if c2.dim() != 2 or c2.shape != (B, DC) or c2.stride(1) != 1:
        raise ValueError("new_c must be [B, kv_lora_rank] with contiguous rows")
    if (R > 0) != (r2 is not None) or (r2 is not None and (r2.shape != (B, R) or r2.stride(1) != 1)):
        raise ValueError("new_rope must be [B, rope_dim] with contiguous rows (None when rope_dim is 0)")
    if r2 is not None and r2.dtype != c2.dtype:
        raise ValueError("new_c and new_rope must share a dtype")
    if new_slots.dtype != torch.int64 or new_slots.numel() != B or not new_slots.is_contiguous():
        raise ValueError("new_slots must be contiguous int64 [B]")
    args = _mla_args(out, q_nope, q_rope, w_uk, w_uv, latent_cache, block_tables, context_lens, softmax_scale,
                     workspace, stream)
    check(lib.pa_mla_decode_step(c2.data_ptr(), c2.stride(0), _ptr(r2), r2.stride(0) if r2 is not None else 0,
                                 _code(c2, "new_c"), new_slots.data_ptr(), *args))
    return out
