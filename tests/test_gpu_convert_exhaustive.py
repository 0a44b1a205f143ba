"""Every fp32 bit pattern through the cache write's conversions, against the oracle.

All 2^32 fp32 bit patterns, in 16 chunks of 2^28 (one fp32 source of 262,144
tokens x 8 heads x 128 dims per chunk, written through an identity slot mapping
so the cache holds the elements in source order), go through
pa_reshape_and_cache into a bf16 cache and into an fp8 e4m3fn cache (no scale).
Each cache is compared bit for bit with the oracle's element encodes of the same
patterns (round to nearest even; bf16 overflow to inf and NaN with sign, top
payload bits and the quiet bit; e4m3fn past 464, infinities and NaN to 0x7F with
the sign). This covers the hardware conversions the write kernel uses for fp32
sources; bf16 sources are covered by the all-65,536-pattern cases of the write
tests."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28
H, D, BS = 8, 128, 16


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _first_mismatch(got, want, src_bits):
    i = int(np.flatnonzero(got != want)[0])
    return f"first mismatch at fp32 bits {int(src_bits[i]):#010x}: gpu {int(got[i]):#x} oracle {int(want[i]):#x}"


def test_every_fp32_pattern_through_the_cache_write():
    import paged_kv_cache_304_amd as pkv
    T = CHUNK // (H * D)
    NB = T // BS
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    src = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    c16 = torch.empty((NB, BS, H, D), dtype=torch.bfloat16, device="cuda")
    c8 = torch.empty((NB, BS, H, D), dtype=torch.float8_e4m3fn, device="cuda")
    for c in range((1 << 32) // CHUNK):
        say(f"fp32 patterns {c * CHUNK:#010x} .. {(c + 1) * CHUNK - 1:#010x}")
        bits = np.arange(c * CHUNK, (c + 1) * CHUNK, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        src.view(-1).copy_(torch.from_numpy(x))
        pkv.reshape_and_cache(src, None, c16, None, slots)
        pkv.reshape_and_cache(src, None, c8, None, slots)
        torch.cuda.synchronize()
        got16 = c16.view(torch.int16).cpu().numpy().view(np.uint16).ravel()
        want16 = oracle.encode_f32_array(x, oracle.BF16)
        assert np.array_equal(got16, want16), "bf16: " + _first_mismatch(got16, want16, bits)
        del got16, want16
        got8 = c8.view(torch.uint8).cpu().numpy().ravel()
        want8 = oracle.encode_f32_array(x, oracle.FP8_E4M3FN)
        assert np.array_equal(got8, want8), "e4m3fn: " + _first_mismatch(got8, want8, bits)
        del got8, want8, bits, x
