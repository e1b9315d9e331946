"""Exhaustive checks of the two shortcuts in the fp8 append arithmetic (fp8_quant.cuh).

1. The row quotient from one reciprocal and one fma correction yields the same e4m3fn code as
   the correctly rounded x / s, for every 16-bit (fp16 and bf16) x with |x| <= absmax and every
   finite 16-bit absmax: this is the whole input domain of the quantiser.
2. The hardware cast v_cvt_pk_fp8_f32 equals the plain integer round-to-nearest-even encoder
   for every fp32 value in [-448, 448], and torch's CPU float8_e4m3fn cast (which the oracle
   is pinned to) for every fp32 value in [0, 448].
3. The decode's conversions of codes back to bf16, fp16 and fp32 values give the oracle's
   e4m3fn value of every one of the 254 non-NaN codes, exactly, for both byte-pair selects.
4. The e5m2 cast v_cvt_pk_bf8_f32 equals the integer round-to-nearest-even encoder for every
   fp32 value in [-57344, 57344], and torch's CPU float8_e5m2 cast on a strided sample; the
   e5m2 and int8 read-side conversions give the oracle's value of every code exactly.

The kernels live in tests/gpu_kernels/fp8_checks.hip and include the library's header, so
the checked code is the code the append kernel runs.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from gpu_helpers import need_gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "gpu_kernels", "libpkv_fp8_checks.so")
MAX_BITS = 0x43E00000       # fp32 bit pattern of 448


def _lib():
    need_gpu()
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built; run paged_kv_cache_45_amd.build.build() first")
    lib = ctypes.CDLL(LIB)
    vp = ctypes.c_void_p
    lib.fp8chk_hw_codes.argtypes = [ctypes.c_uint32, ctypes.c_uint32, vp, vp, vp]
    lib.fp8chk_quotient_codes.argtypes = [ctypes.c_int, vp, vp]
    lib.fp8chk_dequant_codes.argtypes = [vp, vp, vp]
    lib.fp8chk_hw_codes_e5m2.argtypes = [ctypes.c_uint32, ctypes.c_uint32, vp, vp, vp]
    lib.fp8chk_dequant_codes_byte.argtypes = [ctypes.c_int, vp, vp, vp]
    return lib


@pytest.mark.gpu
@pytest.mark.parametrize("bf16", [1, 0])
def test_row_quotient_codes_match_correct_division(bf16):
    lib = _lib()
    bad = torch.zeros(32768 * 256, dtype=torch.int32, device="cuda")
    assert lib.fp8chk_quotient_codes(bf16, bad.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert int(bad.long().sum()) == 0


@pytest.mark.gpu
def test_hardware_cast_matches_rne_and_torch_cpu_cast():
    lib = _lib()
    chunk = 1 << 27
    codes = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    bad = torch.empty(chunk // 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    total_bad = 0
    for u0 in range(0, MAX_BITS + 1, chunk):
        n = min(chunk, MAX_BITS + 1 - u0)
        nt = (n + 255) // 256
        bad.zero_()
        assert lib.fp8chk_hw_codes(u0, nt, codes.data_ptr(), bad.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        total_bad += int(bad.long().sum())
        vals = torch.from_numpy(np.arange(u0, u0 + n, dtype=np.uint32).view(np.float32))
        want = vals.to(torch.float8_e4m3fn).view(torch.uint8)
        got = codes[:n].cpu()
        assert torch.equal(got, want), f"hardware cast differs from torch's CPU cast in [{u0:#x}, {u0 + n:#x})"
    assert total_bad == 0, "hardware cast differs from the integer RNE encoder"


@pytest.mark.gpu
def test_decode_conversions_are_exact_for_every_code():
    from oracle import e4m3fn_decode_table
    lib = _lib()
    out16 = torch.zeros(1024, dtype=torch.int32, device="cuda")
    out32 = torch.zeros(1024, dtype=torch.float32, device="cuda")
    assert lib.fp8chk_dequant_codes(out16.data_ptr(), out32.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    w16 = out16.cpu().numpy().view(np.uint32).reshape(256, 4)
    f32 = out32.cpu().numpy().reshape(256, 4)
    table = e4m3fn_decode_table()                        # float64 [256], NaN for 0x7F / 0xFF
    for c in range(256):
        v = table[c]
        if np.isnan(v):
            assert np.all(np.isnan(f32[c]))
            continue
        bf = np.uint32(np.float32(v).view(np.uint32) >> 16)
        hf = np.uint32(np.float16(v).view(np.uint16))
        assert np.float64(np.float32(v)) == v and np.float64(np.float16(v)) == v   # exact in both
        assert np.all(w16[c, 0:2] == (bf | (bf << 16))), c
        assert np.all(w16[c, 2:4] == (hf | (hf << 16))), c
        assert np.all(f32[c] == np.float32(v)), c


MAX_BITS_E5M2 = 0x47600000  # fp32 bit pattern of 57344


@pytest.mark.gpu
def test_e5m2_hardware_cast_matches_rne_and_torch_cpu_cast():
    lib = _lib()
    chunk = 1 << 27
    codes = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    bad = torch.empty(chunk // 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    total_bad = 0
    for u0 in range(0, MAX_BITS_E5M2 + 1, chunk):
        n = min(chunk, MAX_BITS_E5M2 + 1 - u0)
        nt = (n + 255) // 256
        bad.zero_()
        assert lib.fp8chk_hw_codes_e5m2(u0, nt, codes.data_ptr(), bad.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        total_bad += int(bad.long().sum())
        idx = torch.arange(0, n, 97)
        vals = torch.from_numpy((np.arange(0, n, 97, dtype=np.uint32) + np.uint32(u0)).view(np.float32))
        want = vals.to(torch.float8_e5m2).view(torch.uint8)
        got = codes[:n].cpu()[idx]
        assert torch.equal(got, want), f"e5m2 cast differs from torch's CPU cast in [{u0:#x}, {u0 + n:#x})"
    assert total_bad == 0, "e5m2 cast differs from the integer RNE encoder"


@pytest.mark.gpu
@pytest.mark.parametrize("fmt,kind", [(0, "e5m2"), (1, "i8")])
def test_byte_decode_conversions_are_exact_for_every_code(fmt, kind):
    from oracle import e5m2_decode_table
    lib = _lib()
    out16 = torch.zeros(1024, dtype=torch.int32, device="cuda")
    out32 = torch.zeros(1024, dtype=torch.float32, device="cuda")
    assert lib.fp8chk_dequant_codes_byte(fmt, out16.data_ptr(), out32.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    w16 = out16.cpu().numpy().view(np.uint32).reshape(256, 4)
    f32 = out32.cpu().numpy().reshape(256, 4)
    table = e5m2_decode_table() if kind == "e5m2" else np.arange(256).astype(np.uint8).view(np.int8).astype(np.float64)
    for c in range(256):
        v = table[c]
        if not np.isfinite(v):
            # NaN and infinity codes never occur in a cache the append wrote; the fp32 path
            # still keeps their class
            assert np.all(np.isnan(f32[c])) if np.isnan(v) else np.all(f32[c] == v)
            continue
        bf = np.uint32(np.float32(v).view(np.uint32) >> 16)
        hf = np.uint32(np.float16(v).view(np.uint16))
        assert np.float64(np.float32(v)) == v and np.float64(np.float16(v)) == v
        assert np.float64(np.array([bf << np.uint32(16)], np.uint32).view(np.float32)[0]) == v   # exact in bf16
        assert np.all(w16[c, 0:2] == (bf | (bf << 16))), (kind, c)
        assert np.all(w16[c, 2:4] == (hf | (hf << 16))), (kind, c)
        assert np.all(f32[c] == np.float32(v)), (kind, c)
