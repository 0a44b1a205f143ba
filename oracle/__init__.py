"""CPU oracle for the paged KV cache hot path (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package. The product library neither imports nor links it,
and the two share no code: the arithmetic lives in ``pagedkv_oracle.c`` (plain
C, fp64 for attention, exact bit arithmetic for the encodes), and this module
only marshals numpy arrays into it.

Every function states the passage it follows; the readings R1..R7 and R10 are
listed in the header of ``pagedkv_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pagedkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# PAGEDKV_ORACLE_LIB loads another build of the same source (the CPU sanitizer
# test's AddressSanitizer + UBSan build); it is used as given, never rebuilt.
_LIB_OVERRIDE = os.environ.get("PAGEDKV_ORACLE_LIB")
SANITIZED_LIB = os.path.join(os.path.dirname(_HERE), "_build", "asan", "liboracle.so")

# dtype codes of the C oracle (its own numbering)
BF16, F32, FP8_E4M3FN = 0, 2, 3
_NP_STORAGE = {BF16: np.uint16, F32: np.float32, FP8_E4M3FN: np.uint8}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE arithmetic, no contraction, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized() -> str:
    """The same source compiled with clang's AddressSanitizer and UBSan (shared
    runtime, OpenMP from the same toolchain) into _build/asan/liboracle.so."""
    os.makedirs(os.path.dirname(SANITIZED_LIB), exist_ok=True)
    llvm = "/opt/rocm/llvm"
    cmd = [f"{llvm}/bin/clang", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-shared-libsan", "-fPIC", "-shared", "-Wall", _SRC, "-o", SANITIZED_LIB, "-lm",
           f"-Wl,-rpath,{llvm}/lib"]
    subprocess.run(cmd, check=True)
    return SANITIZED_LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _LIB_OVERRIDE or _LIB_PATH
    if not _LIB_OVERRIDE and (not os.path.exists(_LIB_PATH)
                              or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(path)
    P, I64, I32, F64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = I32
    lib.orc_set_num_threads.argtypes = [I32]
    lib.orc_set_num_threads.restype = None
    lib.orc_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3fn_to_f64.restype = F64
    lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_f32_to_e4m3fn.argtypes = [ctypes.c_float]
    lib.orc_f32_to_e4m3fn.restype = ctypes.c_uint8
    lib.orc_encode_f32_array.argtypes = [P, I64, P, I32]
    lib.orc_encode_f32_array.restype = I32
    lib.orc_encode_bf16_to_fp8_scaled.argtypes = [ctypes.c_uint16, ctypes.c_float]
    lib.orc_encode_bf16_to_fp8_scaled.restype = ctypes.c_uint8
    lib.orc_resolve_slot.argtypes = [P, I64, P, I64, I64]
    lib.orc_resolve_slot.restype = I64
    lib.orc_reshape_and_cache.argtypes = [P, P, I32, I64, I32, I32, I64, I64, P, P, I32, I64, I32,
                                          I64, P, P, I64, P, P]
    lib.orc_reshape_and_cache.restype = I64
    lib.orc_concat_and_cast.argtypes = [P, I32, I64, I64, P, I32, I64, I64, P, I32, I64, I64, I32,
                                        I32, I32]
    lib.orc_concat_and_cast.restype = None
    lib.orc_decode_attention.argtypes = [P, P, I32, I64, P, P, I32, I64, I32, I64, P, I32, P, I32,
                                         I32, I32, I32, F64, P, P]
    lib.orc_decode_attention.restype = None
    lib.orc_prefill_attention.argtypes = [P, P, I32, I64, P, I32, P, P, I32, I64, I32, I64, P, I32,
                                          P, I32, I32, I32, F64, P, P]
    lib.orc_prefill_attention.restype = None
    lib.orc_mla_decode.argtypes = [P, P, I64, P, I64, P, P, P, I64, I32, I64, P, I32, P, I32, I32,
                                   I32, I32, I32, I32, F64]
    lib.orc_mla_decode.restype = None
    _lib = lib
    return lib


def max_threads() -> int:
    """Threads the oracle's parallel loops run with."""
    return int(_load().orc_max_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's parallel loops from now on (timing only)."""
    _load().orc_set_num_threads(int(n))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _scalar_f32(x):
    return None if x is None else np.array([x], dtype=np.float32)


# ------------------------------------------------------------------ encodes

def e4m3fn_to_f64(codes) -> np.ndarray:
    """Value of each OCP e4m3fn code (R4), exactly, as float64."""
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.orc_e4m3fn_to_f64(int(c)) for c in codes], dtype=np.float64)


def f32_to_bf16(x) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (R5)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.orc_f32_to_bf16(float(v)) for v in x], dtype=np.uint16)


def f32_to_e4m3fn(x) -> np.ndarray:
    """fp32 -> e4m3fn code, round to nearest even, overflow/inf/NaN -> signed NaN (R4)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.orc_f32_to_e4m3fn(float(v)) for v in x], dtype=np.uint8)


def encode_f32_array(x, dtype: int) -> np.ndarray:
    """fp32 array -> bf16 bits (uint16) or e4m3fn codes (uint8), one rounding per
    element (R4, R5); OpenMP over the elements."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.shape[0], dtype=np.uint16 if dtype == BF16 else np.uint8)
    if lib.orc_encode_f32_array(_ptr(x), x.shape[0], _ptr(out), dtype) != 0:
        raise ValueError("unsupported dtype")
    return out


def encode_bf16_to_fp8_scaled(bits, scale: float) -> np.ndarray:
    """bf16 bits -> fp32 -> IEEE fp32 division by ``scale`` -> e4m3fn (R3, R4)."""
    lib = _load()
    bits = np.asarray(bits, dtype=np.uint16).ravel()
    s = float(np.float32(scale))
    return np.array([lib.orc_encode_bf16_to_fp8_scaled(int(b), s) for b in bits], dtype=np.uint8)


# ------------------------------------------------------------ slot resolution

def resolve_slots(slot_mapping, num_blocks: int, block_size: int, swa=None) -> np.ndarray:
    """Final slot of every token, -1 for a skipped token (a1; R1, R2)."""
    lib = _load()
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    sw = None if swa is None else np.ascontiguousarray(swa, dtype=np.int64)
    swa_len = 0 if sw is None else sw.shape[0]
    pool = int(num_blocks) * int(block_size)
    return np.array([lib.orc_resolve_slot(_ptr(sm), t, _ptr(sw), swa_len, pool)
                     for t in range(sm.shape[0])], dtype=np.int64)


# --------------------------------------------------------- reshape_and_cache

def reshape_and_cache(key, value, src_dtype: int, key_cache, value_cache, cache_dtype: int,
                      slot_mapping, swa_slot_mapping=None, k_scale=None, v_scale=None,
                      key_token_stride=None, value_token_stride=None) -> int:
    """In-place write of token-major K (and V) into the paged caches (a1, a2).

    ``key``/``value`` are storage arrays (uint16 for bf16, float32, uint8 for
    fp8) viewed as ``[T, ...]`` with the row of token t starting at element
    ``t * token_stride``; the caches are ``[NB, BS, H, D]`` storage arrays
    (contiguous inner ``[BS, H, D]``; the block stride is taken from the array).
    Returns the number of tokens written.
    """
    lib = _load()
    T = int(slot_mapping.shape[0])
    NB, BS, H, D = key_cache.shape
    assert key_cache.dtype == _NP_STORAGE[cache_dtype]
    assert key.dtype == _NP_STORAGE[src_dtype]
    kstride = key_token_stride if key_token_stride is not None else key.strides[0] // key.itemsize
    vstride = 0
    if value is not None:
        vstride = (value_token_stride if value_token_stride is not None
                   else value.strides[0] // value.itemsize)
    block_stride = key_cache.strides[0] // key_cache.itemsize
    assert key_cache.strides[1] // key_cache.itemsize == H * D
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    sw = None if swa_slot_mapping is None else np.ascontiguousarray(swa_slot_mapping,
                                                                     dtype=np.int64)
    ks, vs = _scalar_f32(k_scale), _scalar_f32(v_scale)
    return int(lib.orc_reshape_and_cache(
        _ptr(key), _ptr(value), src_dtype, T, H, D, kstride, vstride,
        _ptr(key_cache), _ptr(value_cache), cache_dtype, NB, BS, block_stride,
        _ptr(sm), _ptr(sw), 0 if sw is None else sw.shape[0], _ptr(ks), _ptr(vs)))


# ------------------------------------------------------------ concat_and_cast

def concat_and_cast(k, k_dtype: int, k_nope, nope_dtype: int, k_rope, rope_dtype: int) -> None:
    """In-place ``k[t,h,:] = cast(cat(k_nope[t,h,:], k_rope[t,0,:]))`` (a3)."""
    lib = _load()
    T, H, KD = k.shape
    nope = k_nope.shape[2]
    rope = k_rope.shape[2]
    assert KD == nope + rope and k_rope.shape[1] == 1 and k_nope.shape[:2] == (T, H)
    for a in (k, k_nope, k_rope):
        assert a.size == 0 or a.strides[2] == a.itemsize
    es = lambda a, i: a.strides[i] // a.itemsize  # noqa: E731
    lib.orc_concat_and_cast(_ptr(k), k_dtype, es(k, 0), es(k, 1), _ptr(k_nope), nope_dtype,
                            es(k_nope, 0), es(k_nope, 1), _ptr(k_rope), rope_dtype, es(k_rope, 0),
                            T, H, nope, rope)


# ---------------------------------------------------------- decode attention

def decode_attention(q, q_dtype: int, key_cache, value_cache, cache_dtype: int, block_tables,
                     context_lens, softmax_scale: float, k_scale=None, v_scale=None,
                     num_kv_heads=None) -> np.ndarray:
    """fp64 single-token paged decode attention, unrounded (a4..a7; R6, R7).

    ``q`` is a ``[B, H_Q, D]`` storage array; caches are ``[NB, BS, H_KV, D]``;
    ``block_tables`` int32 ``[B, W]``; ``context_lens`` int32 ``[B]``.
    """
    lib = _load()
    B, HQ, D = q.shape
    NB, BS, HKV, D2 = key_cache.shape
    assert D == D2 and HQ % HKV == 0
    assert q.strides[1] // q.itemsize == D and q.strides[2] == q.itemsize
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    assert bt.shape[0] == B and cl.shape[0] == B
    block_stride = key_cache.strides[0] // key_cache.itemsize
    assert value_cache.strides == key_cache.strides
    out = np.zeros((B, HQ, D), dtype=np.float64)
    ks, vs = _scalar_f32(k_scale), _scalar_f32(v_scale)
    lib.orc_decode_attention(out.ctypes.data, _ptr(q), q_dtype, q.strides[0] // q.itemsize,
                             _ptr(key_cache), _ptr(value_cache), cache_dtype, NB, BS,
                             block_stride, _ptr(bt), bt.shape[1], _ptr(cl), B, HQ, HKV, D,
                             float(softmax_scale), _ptr(ks), _ptr(vs))
    return out


def prefill_attention(q, q_dtype: int, cu_seqlens_q, key_cache, value_cache, cache_dtype: int,
                      block_tables, context_lens, softmax_scale: float, k_scale=None,
                      v_scale=None) -> np.ndarray:
    """fp64 chunked-prefill paged attention, unrounded (R10).

    ``q`` is a packed ``[T, H_Q, D]`` storage array whose rows cu_seqlens_q[b] ..
    cu_seqlens_q[b+1]-1 are sequence b's queries (the last positions of its
    context); caches are ``[NB, BS, H_KV, D]``; ``block_tables`` int32 ``[B, W]``;
    ``context_lens`` int32 ``[B]``.
    """
    lib = _load()
    T, HQ, D = q.shape
    NB, BS, HKV, D2 = key_cache.shape
    assert D == D2 and HQ % HKV == 0
    assert T == 0 or (q.strides[1] // q.itemsize == D and q.strides[2] == q.itemsize)
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    B = cl.shape[0]
    assert cu.shape[0] == B + 1 and bt.shape[0] == B
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    block_stride = key_cache.strides[0] // key_cache.itemsize
    assert value_cache.strides == key_cache.strides
    out = np.zeros((T, HQ, D), dtype=np.float64)
    ks, vs = _scalar_f32(k_scale), _scalar_f32(v_scale)
    tok_stride = q.strides[0] // q.itemsize if T else HQ * D
    lib.orc_prefill_attention(out.ctypes.data, _ptr(q), q_dtype, tok_stride, _ptr(cu), B,
                              _ptr(key_cache), _ptr(value_cache), cache_dtype, NB, BS,
                              block_stride, _ptr(bt), bt.shape[1], _ptr(cl), HQ, HKV, D,
                              float(softmax_scale), _ptr(ks), _ptr(vs))
    return out


def mla_decode(q_nope, q_rope, w_uk, w_uv, latent_cache, block_tables, context_lens,
               softmax_scale: float) -> np.ndarray:
    """fp64 MLA decode over a latent paged cache with K and V materialised from the
    latent as the page defines them (R13).

    bf16 bit arrays: ``q_nope`` [B, H, qk], ``q_rope`` [B, H, r] (or None for no
    RoPE part), ``w_uk`` [d_c, H*qk], ``w_uv`` [d_c, H*dv], ``latent_cache``
    [NB, BS, d_c + r]; ``block_tables`` int32 [B, W]; ``context_lens`` int32 [B].
    Returns [B, H, dv] fp64."""
    lib = _load()
    B, H, QK = q_nope.shape
    NB, BS, ROW = latent_cache.shape
    R = 0 if q_rope is None else q_rope.shape[2]
    DC = ROW - R
    assert w_uk.shape == (DC, H * QK) and w_uv.shape[0] == DC and w_uv.shape[1] % H == 0
    DV = w_uv.shape[1] // H
    for a in (q_nope, w_uk, w_uv, latent_cache) + (() if q_rope is None else (q_rope,)):
        assert a.dtype == np.uint16
    qn = np.ascontiguousarray(q_nope)
    qr = np.zeros((B, H, 1), dtype=np.uint16) if q_rope is None else np.ascontiguousarray(q_rope)
    wk, wv = np.ascontiguousarray(w_uk), np.ascontiguousarray(w_uv)
    lc = np.ascontiguousarray(latent_cache)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    assert bt.shape[0] == B and cl.shape[0] == B
    out = np.zeros((B, H, DV), dtype=np.float64)
    lib.orc_mla_decode(out.ctypes.data, _ptr(qn), H * QK, _ptr(qr), H * max(R, 1), _ptr(wk), _ptr(wv),
                       _ptr(lc), NB, BS, BS * ROW, _ptr(bt), bt.shape[1], _ptr(cl), B, H, QK, R, DC, DV,
                       float(softmax_scale))
    return out
