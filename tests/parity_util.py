"""Helpers shared by the GPU parity tests: host<->device transfers of raw bit
patterns and the attention tolerance. No arithmetic of the method lives here."""
import numpy as np
import torch

import oracle

TORCH_OF = {oracle.BF16: torch.bfloat16, oracle.F32: torch.float32,
            oracle.FP8_E4M3FN: torch.float8_e4m3fn}
NP_OF = {oracle.BF16: np.uint16, oracle.F32: np.float32, oracle.FP8_E4M3FN: np.uint8}
RAW_VIEW = {oracle.BF16: (torch.int16, np.int16), oracle.F32: (torch.float32, np.float32),
            oracle.FP8_E4M3FN: (torch.uint8, np.uint8)}

# attention tolerance: |gpu - oracle| <= ATOL + RTOL * |oracle|
ATOL = 2e-3
RTOL = 2e-3


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def to_dev(a: np.ndarray, dt: int, device="cuda") -> torch.Tensor:
    """Host storage array (uint16 bf16 bits / float32 / uint8 fp8 codes) -> device tensor."""
    tv, nv = RAW_VIEW[dt]
    t = torch.from_numpy(np.ascontiguousarray(a).view(nv))
    if tv != TORCH_OF[dt]:
        t = t.view(TORCH_OF[dt])
    return t.to(device)


def to_host(t: torch.Tensor, dt: int) -> np.ndarray:
    tv, nv = RAW_VIEW[dt]
    x = t.detach()
    if tv != TORCH_OF[dt]:
        x = x.view(tv)
    return x.cpu().numpy().view(NP_OF[dt])


def sentinel(shape, dt: int, byte: int) -> np.ndarray:
    a = np.empty(shape, dtype=NP_OF[dt])
    a.view(np.uint8)[...] = byte
    return a


def widen_out(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(np.int64) - 8)


def assert_attention_close(gpu: np.ndarray, ref: np.ndarray, what: str = "",
                           out_bf16: bool = True) -> None:
    """|gpu - oracle| <= 2e-3 + 2e-3*|oracle| for fp32 outputs. A bf16 output is one
    more rounding of that fp32 value, so it may also be off by the format's own half
    ulp (which alone exceeds the bound for |oracle| in [2, 2.9) and [4, 5.8))."""
    assert gpu.shape == ref.shape
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    if out_bf16:
        bound = bound + bf16_half_ulp(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} outside tolerance; worst at {i}: "
                             f"gpu={gpu[i]!r} oracle={ref[i]!r} err={err[i]:.3e}")


def abs_values(cache_bits):
    return cache_bits & np.uint16(0x7FFF)   # |x| of bf16 (NaN stays NaN)


def check_close(got, ref, ref_abs, what, out_bf16):
    """Prefill bound: the decode bound plus 2^-9 * sum_j p_j |v_j| / l for the bf16
    probabilities of the P.V product (ref_abs = the oracle run on |V|)."""
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    tol = 2e-3 + 2e-3 * np.abs(ref) + 2.0 ** -9 * ref_abs * 1.001
    if out_bf16:
        tol = tol + bf16_half_ulp(ref)
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside the bound; worst at {i}: "
                             f"gpu {got[i]!r} oracle {ref[i]!r} tol {tol[i]!r}")
