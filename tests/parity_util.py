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
    """|gpu - oracle| <= 2e-3 + 2e-3*|oracle| against the unrounded fp64 oracle.

    A bf16 output is one more rounding of the kernel's fp32 value. Below |oracle| = 2
    that rounding stays inside the bound (half an ulp is at most 2^-8 * |oracle|, and
    at most 2^-9 * 2 there), so the plain bound applies. Only where |oracle| >= 2
    can bf16's half ulp alone exceed it (|oracle| in [2, 2.9) and [4, 5.8)); there,
    and only there, half an ulp of the oracle value is added, and the test says how
    many outputs took that allowance."""
    assert gpu.shape == ref.shape
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    if out_bf16:
        big = np.abs(ref) >= 2.0
        if big.any():
            say(f"{what}: {int(big.sum())} of {ref.size} outputs have |o| >= 2 "
                f"(bf16 half-ulp allowance applied to those only)")
            bound = bound + np.where(big, bf16_half_ulp(ref), 0.0)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} outside tolerance; worst at {i}: "
                             f"gpu={gpu[i]!r} oracle={ref[i]!r} err={err[i]:.3e}")
