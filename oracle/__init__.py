"""fp64 CPU oracle for paged-KV decode -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use this package; the product path never does.  It wraps
``oracle.c`` (plain C, built with gcc into ``liboracle.so``) through ctypes and
shares nothing with the HIP library.

Inputs are host tensors or arrays holding the *stored* bytes (torch CPU
tensors of dtype float32 / float16 / bfloat16 / float8_e4m3fn, int32 tables and
lengths, int64 slot mappings).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

ORC_F32, ORC_F16, ORC_BF16, ORC_FP8 = 0, 1, 2, 3
STATUS = {
    0: "ok",
    1: "bad argument",
    2: "block id outside the pool",
    3: "context longer than the table row",
    4: "slot outside the pool",
    5: "duplicate slot",
    6: "out of memory",
}


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall",
                               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            i64, i32, vp, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
            lib.oracle_paged_decode.restype = i32
            lib.oracle_paged_decode.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp] + [i64] * 7 + [dbl] * 3 + \
                [vp, vp, vp, vp, i32]
            lib.oracle_paged_prefill.restype = i32
            lib.oracle_paged_prefill.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp, vp] + [i64] * 7 + [dbl] * 3 + \
                [vp, vp, vp, vp, i32]
            lib.oracle_cache_write.restype = i32
            lib.oracle_cache_write.argtypes = [vp, vp, i32, vp, vp, i32, vp] + [i64] * 5 + [ctypes.c_float] * 2 + \
                [vp, vp, vp, vp]
            lib.oracle_f16_to_double.restype = dbl
            lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_bf16_to_double.restype = dbl
            lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_fp8_to_double.restype = dbl
            lib.oracle_fp8_to_double.argtypes = [ctypes.c_uint8]
            lib.oracle_float_to_fp8.restype = ctypes.c_uint8
            lib.oracle_float_to_fp8.argtypes = [ctypes.c_float]
            _lib = lib
    return _lib


def _code(t) -> int:
    import torch

    return {
        torch.float32: ORC_F32,
        torch.float16: ORC_F16,
        torch.bfloat16: ORC_BF16,
        torch.float8_e4m3fn: ORC_FP8,
    }[t.dtype]


def _host(t, dtype=None):
    import torch

    if isinstance(t, np.ndarray):
        t = torch.from_numpy(t)
    t = t.detach().to("cpu")
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous()


def _scales(k_scale, v_scale, count: int, dtype, num_blocks: int = 0):
    """(per-tensor k, per-tensor v, per-head k, per-head v, per-block k,
    per-block v): scalars are per-tensor fp8 scales, sequences of ``count``
    values one scale per kv head, [num_blocks, count] arrays one scale per
    (physical block, kv head); the arrays not given are None."""
    if np.ndim(k_scale) == 0 and np.ndim(v_scale) == 0:
        return float(k_scale), float(v_scale), None, None, None, None
    ka = np.ascontiguousarray(np.asarray(_host_array(k_scale), dtype=dtype))
    va = np.ascontiguousarray(np.asarray(_host_array(v_scale), dtype=dtype))
    if ka.ndim == 2 or va.ndim == 2:
        if ka.shape != (num_blocks, count) or va.shape != (num_blocks, count):
            raise ValueError(f"per-block scales need [{num_blocks}, {count}] values each")
        return 1.0, 1.0, None, None, ka, va
    ka, va = ka.reshape(-1), va.reshape(-1)
    if ka.shape[0] != count or va.shape[0] != count:
        raise ValueError(f"per-head scales need {count} values each")
    return 1.0, 1.0, ka, va, None, None


def _ptr(a):
    return None if a is None else a.ctypes.data


def _host_array(x):
    import torch

    return x.detach().cpu().numpy() if torch.is_tensor(x) else x


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, num_kv_heads: int,
                 k_scale=1.0, v_scale=1.0, nthreads: int = 1) -> np.ndarray:
    """Reference decode; returns float64 [num_seqs, num_heads, head_dim].

    ``k_scale`` / ``v_scale`` (fp8 caches): one scale per tensor, a sequence
    of num_kv_heads scales (one per kv head), or a [num_blocks, num_kv_heads]
    array (one per physical block and kv head)."""
    import torch

    lib = _load()
    q, k_cache, v_cache = _host(q), _host(k_cache), _host(v_cache)
    bt = _host(block_tables, torch.int32)
    cl = _host(context_lens, torch.int32)
    S, H, D = q.shape
    NB, bs, Hkv, Dk = k_cache.shape
    if Hkv != num_kv_heads or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shape does not match q / num_kv_heads")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache dtypes differ")
    W = bt.shape[1] if bt.dim() == 2 else 0
    ks, vs, kh, vh, kb, vb = _scales(k_scale, v_scale, Hkv, np.float64, NB)
    out = np.empty((S, H, D), dtype=np.float64)
    rc = lib.oracle_paged_decode(out.ctypes.data, q.data_ptr(), _code(q), k_cache.data_ptr(), v_cache.data_ptr(),
                                 _code(k_cache), bt.data_ptr(), cl.data_ptr(), S, H, Hkv, D, NB, bs, W,
                                 float(scale), ks, vs, _ptr(kh), _ptr(vh), _ptr(kb), _ptr(vb), int(nthreads))
    if rc != 0:
        raise OracleError(f"oracle_paged_decode: {STATUS.get(rc, rc)}")
    return out


def paged_decode_layers(q, k_caches, v_caches, block_tables, context_lens, scale: float, num_kv_heads: int,
                        k_scale=1.0, v_scale=1.0, nthreads: int = 1):
    """Reference decode of several layers of one batch: [L, S, H, D] float64.

    Every layer has its own queries and caches ([L, ...] tensors) and they all
    share one set of block tables and context lengths, since block b names the
    same tokens in every layer's pool.  Layer l is exactly paged_decode on
    layer l's tensors; batching the layers changes nothing in what is computed
    (page "vLLM框架中的KV cache优化与PagedAttention机制详解", section 5.2, batches
    the translation of many lookups into one call)."""
    L = q.shape[0]
    if k_caches.shape[0] != L or v_caches.shape[0] != L:
        raise ValueError("q, k_caches and v_caches must have the same number of layers")
    per_head = np.ndim(k_scale) > 0
    if per_head:  # [L, num_kv_heads] or [L, num_blocks, num_kv_heads]: layer l's part
        k_scale = np.asarray(_host_array(k_scale), dtype=np.float64)
        v_scale = np.asarray(_host_array(v_scale), dtype=np.float64)
        if k_scale.ndim != 3:
            k_scale, v_scale = k_scale.reshape(L, num_kv_heads), v_scale.reshape(L, num_kv_heads)
    return np.stack([paged_decode(q[l], k_caches[l], v_caches[l], block_tables, context_lens, scale, num_kv_heads,
                                  k_scale[l] if per_head else k_scale, v_scale[l] if per_head else v_scale,
                                  nthreads) for l in range(L)]) if L else \
        np.zeros(tuple(q.shape), dtype=np.float64)


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale: float,
                  num_kv_heads: int, k_scale=1.0, v_scale=1.0, nthreads: int = 1) -> np.ndarray:
    """Reference prefill (causal, the query rows of sequence s being its newest
    query_start_loc[s+1] - query_start_loc[s] tokens); returns float64
    [num_query_rows, num_heads, head_dim]."""
    import torch

    lib = _load()
    q, k_cache, v_cache = _host(q), _host(k_cache), _host(v_cache)
    bt = _host(block_tables, torch.int32)
    cl = _host(context_lens, torch.int32)
    qsl = _host(query_start_loc, torch.int32)
    N, H, D = q.shape
    NB, bs, Hkv, Dk = k_cache.shape
    S = cl.shape[0]
    if Hkv != num_kv_heads or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shape does not match q / num_kv_heads")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache dtypes differ")
    if qsl.shape[0] != S + 1 or int(qsl[-1]) != N:
        raise ValueError("query_start_loc must have num_seqs + 1 entries ending at the query row count")
    W = bt.shape[1] if bt.dim() == 2 else 0
    ks, vs, kh, vh, kb, vb = _scales(k_scale, v_scale, Hkv, np.float64, NB)
    out = np.empty((N, H, D), dtype=np.float64)
    rc = lib.oracle_paged_prefill(out.ctypes.data, q.data_ptr(), _code(q), k_cache.data_ptr(), v_cache.data_ptr(),
                                  _code(k_cache), bt.data_ptr(), cl.data_ptr(), qsl.data_ptr(), S, H, Hkv, D, NB,
                                  bs, W, float(scale), ks, vs, _ptr(kh), _ptr(vh), _ptr(kb), _ptr(vb),
                                  int(nthreads))
    if rc != 0:
        raise OracleError(f"oracle_paged_prefill: {STATUS.get(rc, rc)}")
    return out


def cache_write(k, v, k_cache, v_cache, slot_mapping, k_scale=1.0, v_scale=1.0,
                inplace: bool = False):
    """Reference cache write; returns (k_cache, v_cache) as CPU tensors.

    With ``inplace`` the given contiguous CPU caches are updated and returned;
    otherwise host copies are made first."""
    import torch

    lib = _load()
    k, v = _host(k), _host(v)
    if inplace:
        kc, vc = k_cache, v_cache
        if kc.device.type != "cpu" or not kc.is_contiguous() or not vc.is_contiguous():
            raise ValueError("inplace cache_write needs contiguous CPU caches")
    else:
        kc, vc = _host(k_cache).clone(), _host(v_cache).clone()
    sm = _host(slot_mapping, torch.int64)
    N, Hkv, D = k.shape
    NB, bs = kc.shape[0], kc.shape[1]
    ks, vs, kh, vh, kb, vb = _scales(k_scale, v_scale, Hkv, np.float32, NB)
    rc = lib.oracle_cache_write(k.data_ptr(), v.data_ptr(), _code(k), kc.data_ptr(), vc.data_ptr(), _code(kc),
                                sm.data_ptr(), N, Hkv, D, NB, bs, ks, vs, _ptr(kh), _ptr(vh), _ptr(kb), _ptr(vb))
    if rc != 0:
        raise OracleError(f"oracle_cache_write: {STATUS.get(rc, rc)}")
    return kc, vc


def copy_blocks(dst_cache, src_cache, block_mapping, inplace: bool = False):
    """Reference block copy; returns the destination pool as a CPU tensor.

    For every pair (s, d) of ``block_mapping`` ([M, 2]), block d of the
    destination pool becomes a byte copy of block s of the source pool.  This
    is the copy that a write into a shared, partly filled block needs first
    (page "vLLM框架中的KV cache优化与PagedAttention机制详解", section 5.1, step 4:
    shared blocks are copied before they are modified), and the move of whole
    blocks between GPU and CPU memory (page "Paged KVCache：大模型推理显存管理优化方案",
    section 5, blocks migrating between memory tiers).  A pair with a negative
    id is skipped.  Raises OracleError for an id past its pool, a destination
    named twice, or -- when both pools are the same tensor -- a destination
    that is also a source (the result would depend on the order of copies).
    Pools are [num_blocks, ...] of any dtype; only bytes move."""
    import torch

    same = dst_cache is src_cache or (dst_cache.data_ptr() == src_cache.data_ptr()
                                      and dst_cache.device == src_cache.device)
    src = _host(src_cache)
    if inplace:
        dst = dst_cache
        if dst.device.type != "cpu" or not dst.is_contiguous():
            raise ValueError("inplace copy_blocks needs a contiguous CPU pool")
    else:
        dst = _host(dst_cache).clone()
    if same:
        src = dst
    if tuple(src.shape[1:]) != tuple(dst.shape[1:]) or src.dtype != dst.dtype:
        raise ValueError("pools differ in block shape or dtype")
    pairs = [(int(a), int(b)) for a, b in _host(block_mapping, torch.int64).reshape(-1, 2).tolist()]
    live = [(a, b) for a, b in pairs if a >= 0 and b >= 0]
    for a, b in live:
        if a >= src.shape[0] or b >= dst.shape[0]:
            raise OracleError("copy_blocks: block id outside the pool")
    dsts = [b for _, b in live]
    if len(set(dsts)) != len(dsts):
        raise OracleError("copy_blocks: a destination block is named twice")
    if same and set(dsts) & {a for a, _ in live}:
        raise OracleError("copy_blocks: a destination block is also a source")
    sb = src.view(torch.uint8).reshape(src.shape[0], -1)
    db = dst.view(torch.uint8).reshape(dst.shape[0], -1)
    for a, b in live:
        db[b] = sb[a]
    return dst


def f16_to_double(bits: int) -> float:
    return _load().oracle_f16_to_double(bits)


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(bits)


def fp8_to_double(code: int) -> float:
    return _load().oracle_fp8_to_double(code)


def float_to_fp8(x: float) -> int:
    return int(_load().oracle_float_to_fp8(x))
