"""paged_kv_cache_45_amd - paged KV cache hot path for AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/pagedkv.h (libpagedkv.so, built in-tree
by `paged_kv_cache_45_amd.build`).  The functions here only marshal torch tensors
into pointers, strides and sizes and call the library; every step of the path runs
in the HIP kernels.  There is no fallback: if the library is missing or a call fails,
an exception is raised.

Entry points (same names as the C ABI):
    kv_append, kv_append_scaled, paged_decode, paged_decode_scaled, paged_decode_append, paged_decode_noalloc,
    paged_decode_workspace_size, build_slot_mapping, pack3, unpack3, pkv_status_string
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = ["kv_append", "kv_append_scaled", "paged_decode", "paged_decode_scaled", "paged_decode_append",
           "paged_decode_noalloc",
           "build_slot_mapping", "paged_decode_workspace_size", "pack3", "unpack3",
           "pkv_status_string", "decode_workspace", "library_path", "load_library",
           "PKV_F16", "PKV_BF16", "PKV_FP8_E4M3FN", "PKV_U3", "PKV_FP8_E5M2", "PKV_INT8",
           "PagedKVError"]

PKV_F16, PKV_BF16, PKV_FP8_E4M3FN, PKV_U3, PKV_FP8_E5M2, PKV_INT8 = 0, 1, 2, 3, 4, 5
_STATUS = {0: "PKV_OK", -1: "PKV_EINVAL", -2: "PKV_EUNSUPPORTED", -3: "PKV_EWORKSPACE",
           -4: "PKV_EHIP", -5: "PKV_ESCRATCH"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class PagedKVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} ({pkv_status_string(status)})")


def library_path() -> str:
    return os.path.join(_HERE, "libpagedkv.so")


def load_library() -> ctypes.CDLL:
    """Load libpagedkv.so.  torch is imported first so that the library binds to the HIP
    runtime torch already loaded (same soname), and shares its streams."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  (loads torch's HIP runtime before ours)
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run paged_kv_cache_45_amd.build.build() "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    i64, i32, vp, f32, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    lib.kv_append.restype = i32
    lib.kv_append.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, i64, vp, vp, i32, i64, i64, i64,
                              vp, vp, i64, i32, i32, i32, vp]
    lib.kv_append_scaled.restype = i32
    lib.kv_append_scaled.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, i64, vp, vp, i32, i64, i64,
                                     i64, vp, vp, i64, i64, i64, i64, i32, i32, i32, vp]
    lib.paged_decode_workspace_size.restype = sz
    lib.paged_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.paged_decode.restype = i32
    lib.paged_decode.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, i32, i64, i64, i64, vp, vp,
                                 vp, i64, vp, i32, i32, i32, i32, i32, i64, i32, f32, i32, vp, sz, vp]
    lib.paged_decode_scaled.restype = i32
    lib.paged_decode_scaled.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, i32, i64, i64, i64,
                                        vp, vp, i64, i64, i64, vp, i64, vp, i32, i32, i32, i32, i32,
                                        i64, i32, f32, i32, vp, sz, vp]
    lib.paged_decode_append.restype = i32
    lib.paged_decode_append.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, i64, i64, i64, i64,
                                        vp, vp, i32, i64, i64, i64, vp, vp, vp, i64, vp, i32, i32, i32,
                                        i32, i32, i64, i32, f32, i32, vp, sz, vp]
    lib.paged_decode_noalloc.restype = i32
    lib.paged_decode_noalloc.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, i32, i64, i64, i64,
                                         vp, vp, vp, i64, vp, i32, i32, i32, i32, i32, i64, i32, f32,
                                         i32, vp]
    lib.build_slot_mapping.restype = i32
    lib.build_slot_mapping.argtypes = [vp, vp, i64, vp, i64, i32, i32, vp, vp]
    lib.pack3.restype = i32
    lib.pack3.argtypes = [vp, vp, i64, vp]
    lib.unpack3.restype = i32
    lib.unpack3.argtypes = [vp, vp, i64, vp]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [i32]
    _LIB = lib
    return lib


def pkv_status_string(status: int) -> str:
    return load_library().pkv_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PagedKVError(fn, status)


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype16(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return PKV_F16
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise TypeError(f"expected float16 or bfloat16, got {t.dtype}")


def _cache_dtype(cache, ref_dtype: int, cache_dtype) -> int:
    import torch
    if cache_dtype is not None:
        return {"same": ref_dtype, "fp8": PKV_FP8_E4M3FN, "e5m2": PKV_FP8_E5M2, "i8": PKV_INT8,
                "u3": PKV_U3}.get(cache_dtype, cache_dtype)
    if cache.dtype in (torch.float16, torch.bfloat16):
        return _dtype16(cache)
    if cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PKV_FP8_E4M3FN
    if cache.dtype == torch.float8_e5m2:
        return PKV_FP8_E5M2
    if cache.dtype == torch.int8:
        return PKV_INT8
    if cache.dtype in (torch.int32, torch.uint32):
        return PKV_U3
    raise TypeError(f"cannot infer the cache dtype from {cache.dtype}")


def _cache_strides(k_cache, v_cache):
    if k_cache.dim() != 4 or k_cache.stride(3) != 1:
        raise ValueError("caches must be [num_blocks, block_size, num_kv_heads, row] with unit row stride")
    if tuple(k_cache.stride()) != tuple(v_cache.stride()) or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    return k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, k_meta=None, v_meta=None,
              cache_dtype=None, stream=None, scale_strides=None) -> None:
    """Write new K/V [T, Hkv, D] into the paged pools through slot_mapping (int64 [T]).

    Caches: [NB, BS, Hkv, D] (same dtype as the input, or byte codes - fp8 e4m3fn, fp8 e5m2
    or int8, named by cache_dtype "fp8" / "e5m2" / "i8" or by the tensor's dtype - with fp32
    meta [NB, BS, Hkv]) or [NB, BS, Hkv, 3*D/32] int32 3-bit words with fp16 meta
    [NB, BS, Hkv, 2].

    scale_strides=(sb, ss, sh): byte-code caches with caller-given fp32 scales (kv_append_scaled):
    k_meta / v_meta are then read, never written, at blk*sb + slot*ss + head*sh."""
    in_dt = _dtype16(k_new)
    if k_new.dim() != 3 or v_new.shape != k_new.shape or k_new.stride(2) != 1 or v_new.stride(2) != 1:
        raise ValueError("k_new / v_new must be [T, Hkv, D] with unit stride on D")
    cdt = _cache_dtype(k_cache, in_dt, cache_dtype)
    sb, ss, sh = _cache_strides(k_cache, v_cache)
    T, H, D = k_new.shape
    lib = load_library()
    if scale_strides is not None:
        st = lib.kv_append_scaled(
            _ptr(k_new), _ptr(v_new), in_dt, k_new.stride(0), k_new.stride(1), v_new.stride(0),
            v_new.stride(1), _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache), cdt, sb, ss, sh,
            _ptr(k_meta), _ptr(v_meta), *(int(v) for v in scale_strides), k_cache.shape[0],
            k_cache.shape[1], H, D, _stream(stream))
        _check("kv_append_scaled", st)
        return
    st = lib.kv_append(
        _ptr(k_new), _ptr(v_new), in_dt, k_new.stride(0), k_new.stride(1), v_new.stride(0),
        v_new.stride(1), _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache), cdt, sb, ss, sh,
        _ptr(k_meta), _ptr(v_meta), k_cache.shape[0], k_cache.shape[1], H, D, _stream(stream))
    _check("kv_append", st)


def paged_decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                max_context_len: int, partition_size: int = 0) -> int:
    n = load_library().paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                                   max_context_len, partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid arguments to paged_decode_workspace_size")
    return int(n)


def decode_workspace(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     max_context_len: int, partition_size: int = 0, device="cuda"):
    """Allocate the workspace paged_decode needs on `device` (None if none).  Its contents do
    not matter: every call writes what it reads."""
    import torch
    n = paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                    partition_size)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                 sm_scale: Optional[float] = None, k_meta=None, v_meta=None, partition_size: int = 0,
                 workspace=None, out=None, cache_dtype=None, head_dim: Optional[int] = None,
                 stream=None, scale_strides=None):
    """Single-query paged attention: q [B, Hq, D] -> out [B, Hq, D] (q's dtype).

    scale_strides=(sb, ss, sh): byte-code caches with caller-given fp32 scales
    (paged_decode_scaled), k_meta / v_meta read at blk*sb + slot*ss + head*sh."""
    import torch
    qdt = _dtype16(q)
    if q.dim() != 3 or q.stride(2) != 1:
        raise ValueError("q must be [B, Hq, D] with unit stride on D")
    B, Hq, D = q.shape
    cdt = _cache_dtype(k_cache, qdt, cache_dtype)
    sb, ss, sh = _cache_strides(k_cache, v_cache)
    if out is None:
        out = torch.empty_like(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be [B, max_blocks] with unit stride")
    if workspace is None:
        workspace = decode_workspace(B, Hq, k_cache.shape[2], D, max_context_len, partition_size,
                                     q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    tail = (_ptr(block_tables), block_tables.stride(0), _ptr(context_lens), B, Hq, k_cache.shape[2], D,
            k_cache.shape[1], k_cache.shape[0], int(max_context_len), float(sm_scale),
            int(partition_size), _ptr(workspace), wbytes, _stream(stream))
    head = (_ptr(out), _ptr(q), qdt, q.stride(0), q.stride(1), out.stride(0), out.stride(1),
            _ptr(k_cache), _ptr(v_cache), cdt, sb, ss, sh, _ptr(k_meta), _ptr(v_meta))
    if scale_strides is not None:
        st = load_library().paged_decode_scaled(*head, *(int(v) for v in scale_strides), *tail)
        _check("paged_decode_scaled", st)
    else:
        st = load_library().paged_decode(*head, *tail)
        _check("paged_decode", st)
    return out


def paged_decode_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                        max_context_len: int, sm_scale: Optional[float] = None, k_meta=None,
                        v_meta=None, partition_size: int = 0, workspace=None, out=None,
                        cache_dtype=None, stream=None):
    """One decode step in one launch: k_new / v_new [B, Hkv, D] (q's dtype) appended at position
    context_lens[b] - 1 of each request (the slot from its block table; none where the length is
    0), then paged_decode over context_lens (which count the new token)."""
    import torch
    qdt = _dtype16(q)
    if q.dim() != 3 or q.stride(2) != 1:
        raise ValueError("q must be [B, Hq, D] with unit stride on D")
    B, Hq, D = q.shape
    for t in (k_new, v_new):
        if t.dim() != 3 or t.stride(2) != 1 or t.dtype != q.dtype or tuple(t.shape) != (B, k_cache.shape[2], D):
            raise ValueError("k_new / v_new must be [B, Hkv, D] of q's dtype with unit stride on D")
    cdt = _cache_dtype(k_cache, qdt, cache_dtype)
    sb, ss, sh = _cache_strides(k_cache, v_cache)
    if out is None:
        out = torch.empty_like(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be [B, max_blocks] with unit stride")
    if workspace is None:
        workspace = decode_workspace(B, Hq, k_cache.shape[2], D, max_context_len, partition_size,
                                     q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().paged_decode_append(
        _ptr(out), _ptr(q), qdt, q.stride(0), q.stride(1), out.stride(0), out.stride(1),
        _ptr(k_new), _ptr(v_new), k_new.stride(0), k_new.stride(1), v_new.stride(0), v_new.stride(1),
        _ptr(k_cache), _ptr(v_cache), cdt, sb, ss, sh, _ptr(k_meta), _ptr(v_meta),
        _ptr(block_tables), block_tables.stride(0), _ptr(context_lens), B, Hq, k_cache.shape[2], D,
        k_cache.shape[1], k_cache.shape[0], int(max_context_len), float(sm_scale),
        int(partition_size), _ptr(workspace), wbytes, _stream(stream))
    _check("paged_decode_append", st)
    return out


def paged_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                         sm_scale: Optional[float] = None, k_meta=None, v_meta=None,
                         partition_size: int = 0, out=None, cache_dtype=None, stream=None):
    """paged_decode with the library's static device scratch in place of a workspace (the
    library allocates nothing; the caller passes q, the caches and out).  Calls that overlap on
    one GPU share the scratch and race."""
    import torch
    qdt = _dtype16(q)
    if q.dim() != 3 or q.stride(2) != 1:
        raise ValueError("q must be [B, Hq, D] with unit stride on D")
    B, Hq, D = q.shape
    cdt = _cache_dtype(k_cache, qdt, cache_dtype)
    sb, ss, sh = _cache_strides(k_cache, v_cache)
    if out is None:
        out = torch.empty_like(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be [B, max_blocks] with unit stride")
    st = load_library().paged_decode_noalloc(
        _ptr(out), _ptr(q), qdt, q.stride(0), q.stride(1), out.stride(0), out.stride(1),
        _ptr(k_cache), _ptr(v_cache), cdt, sb, ss, sh, _ptr(k_meta), _ptr(v_meta),
        _ptr(block_tables), block_tables.stride(0), _ptr(context_lens), B, Hq, k_cache.shape[2], D,
        k_cache.shape[1], k_cache.shape[0], int(max_context_len), float(sm_scale),
        int(partition_size), _stream(stream))
    _check("paged_decode_noalloc", st)
    return out


def kv_append_scaled(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, scale_strides,
                     cache_dtype=None, stream=None) -> None:
    """kv_append into a byte-code cache with the caller's fp32 scales (read only), the scale of
    row (blk, slot, head) at blk*sb + slot*ss + head*sh for scale_strides = (sb, ss, sh)."""
    kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, cache_dtype=cache_dtype,
              stream=stream, scale_strides=scale_strides)


def paged_decode_scaled(q, k_cache, v_cache, k_scale, v_scale, scale_strides, block_tables,
                        context_lens, max_context_len: int, **kw):
    """paged_decode over a byte-code cache with caller-given scales (see kv_append_scaled)."""
    return paged_decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                        k_meta=k_scale, v_meta=v_scale, scale_strides=scale_strides, **kw)


def build_slot_mapping(token_position, block_size: int, batch: int, block_tables=None,
                       token_request=None, out=None, stream=None):
    """int64 slot ids [T] of new tokens from int32 positions [T] (and int32 requests [T], or
    None for request t = token t): paged through block_tables [batch, max_blocks], or the
    contiguous cache's request * block_size + position without a table; -1 for padding."""
    import torch
    T = token_position.numel()
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=token_position.device)
    bts = 0 if block_tables is None else block_tables.stride(0)
    st = load_library().build_slot_mapping(_ptr(token_request), _ptr(token_position), T,
                                           _ptr(block_tables), bts, int(batch), int(block_size),
                                           _ptr(out), _stream(stream))
    _check("build_slot_mapping", st)
    return out


def pack3(values, packed=None, stream=None):
    """uint8 values [n] (n % 8 == 0, low 3 bits used) -> uint8 packed [3n/8]."""
    import torch
    n = values.numel()
    if packed is None:
        packed = torch.empty(3 * n // 8, dtype=torch.uint8, device=values.device)
    _check("pack3", load_library().pack3(_ptr(values), _ptr(packed), n, _stream(stream)))
    return packed


def unpack3(packed, n_values: Optional[int] = None, values=None, stream=None):
    """uint8 packed [3n/8] -> uint8 values [n] in 0..7."""
    import torch
    n = packed.numel() * 8 // 3 if n_values is None else int(n_values)
    if values is None:
        values = torch.empty(n, dtype=torch.uint8, device=packed.device)
    _check("unpack3", load_library().unpack3(_ptr(packed), _ptr(values), n, _stream(stream)))
    return values
