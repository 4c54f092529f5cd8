"""Thin Python binding of libmimo_attn.so (argument marshalling only).

Functions carry the C ABI's names and take torch tensors on the GPU: bf16
tensors for q/k/v/out/caches, int64 for positions, float32 for sinks / lse.
Each call passes data_ptr()s and torch's current HIP stream to the library;
every step of the computation runs in the library's kernels.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmimo_attn.so")

MIMO_OK = 0
_STATUS = {1: "MIMO_ERR_INVALID_ARGUMENT", 2: "MIMO_ERR_UNSUPPORTED", 3: "MIMO_ERR_WORKSPACE",
           4: "MIMO_ERR_HIP"}


class MimoAttnCfg(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("rope_base", ctypes.c_double),
                ("softmax_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("window", ctypes.c_int32)]


def swa_cfg(window: int = 128) -> MimoAttnCfg:
    """Sliding-window layer: 64 q heads / 8 KV heads, base 1e4, window 128."""
    return MimoAttnCfg(64, 8, 192, 128, 64, 1.0e4, 1.0 / math.sqrt(192.0), 0.707, window)


def global_cfg() -> MimoAttnCfg:
    """Global layer: 64 q heads / 4 KV heads, base 1e7, no window."""
    return MimoAttnCfg(64, 4, 192, 128, 64, 1.0e7, 1.0 / math.sqrt(192.0), 0.707, 0)


class MimoError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the built library (it is never built implicitly here)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with global_attention_sinks_amd.build.build()")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    C = ctypes.POINTER(MimoAttnCfg)
    lib.mimo_rope_partial.argtypes = [C, P, P, I64, I32, P, P]
    lib.mimo_attn_prefill_swa.argtypes = [C, P, P, P, P, I32, I32, I64, P, P, P]
    lib.mimo_attn_prefill_global.argtypes = [C, P, P, P, I32, I32, I32, I64, P, P, P, ctypes.c_size_t, P]
    lib.mimo_attn_prefill_varlen.argtypes = [C, P, P, P, P, I32, P, P, P, I32, I32, I64, P, P, P,
                                             ctypes.c_size_t, P]
    lib.mimo_attn_prefill_workspace_size.argtypes = [C, I32, I64]
    lib.mimo_attn_prefill_workspace_size.restype = ctypes.c_size_t
    lib.mimo_attn_decode.argtypes = [C, I32, P, P, P, P, I32, P, P, P, ctypes.c_size_t, P]
    lib.mimo_attn_decode_noalloc.argtypes = [C, I32, P, P, P, P, I32, P, P, P]
    lib.mimo_attn_prefill_backward.argtypes = [C, P, P, P, P, I32, I32, I64, P, P, P, P, P, P, P, P,
                                               ctypes.c_size_t, P]
    lib.mimo_attn_backward_workspace_size.argtypes = [C, I32, I32]
    lib.mimo_attn_backward_workspace_size.restype = ctypes.c_size_t
    lib.mimo_attn_decode_workspace_size.argtypes = [C, I32, I32]
    lib.mimo_attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.mimo_attn_decode_multi.argtypes = [C, I32, I32, P, P, P, P, I32, P, P, P, ctypes.c_size_t, P]
    F = ctypes.c_float
    lib.mimo_attn_decode_paged.argtypes = [C, I32, I32, P, P, P, P, I32, I32, ctypes.c_int, F, F, P, I32, P, P, P,
                                           ctypes.c_size_t, P]
    lib.mimo_kv_paged_append.argtypes = [C, I32, P, P, P, P, P, I32, I32, ctypes.c_int, F, F, P, I32, P]
    lib.mimo_attn_decode_multi_workspace_size.argtypes = [C, I32, I32, I32]
    lib.mimo_attn_decode_multi_workspace_size.restype = ctypes.c_size_t
    lib.mimo_kv_ring_append.argtypes = [C, I32, P, P, P, P, P, I32, P]
    lib.mimo_last_error.restype = ctypes.c_char_p
    for fn in ("mimo_rope_partial", "mimo_attn_prefill_swa", "mimo_attn_prefill_global",
               "mimo_attn_prefill_varlen", "mimo_attn_decode", "mimo_attn_decode_noalloc", "mimo_attn_decode_multi",
               "mimo_attn_decode_paged", "mimo_kv_paged_append", "mimo_kv_ring_append",
               "mimo_attn_prefill_backward"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != MIMO_OK:
        raise MimoError(fn, status, _lib.mimo_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name, ndim=None):
    if t is None:
        return
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _shape(t, name, *dims):
    """Every tensor's full shape is checked against the call's sizes, so that no kernel
    indexes past a tensor the caller made too small."""
    if t is not None and tuple(t.shape) != dims:
        raise ValueError(f"{name} must have shape {dims}, got {tuple(t.shape)}")


def _ws(ws):
    if ws is None:
        return 0
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous CUDA tensor")
    return ws.numel() * ws.element_size()


def mimo_rope_partial(cfg: MimoAttnCfg, x_in, x_out, pos, stream=None):
    """x_in/x_out [n_tokens, n_heads, 192] bf16 (may be the same tensor), pos [n_tokens] int64."""
    lib = load_library()
    _need(x_in, torch.bfloat16, "x_in", 3); _need(x_out, torch.bfloat16, "x_out", 3)
    _need(pos, torch.int64, "pos", 1)
    n, h, _ = x_in.shape
    _shape(x_in, "x_in", n, h, 192); _shape(x_out, "x_out", n, h, 192); _shape(pos, "pos", n)
    _check("mimo_rope_partial", lib.mimo_rope_partial(ctypes.byref(cfg), _p(x_in), _p(x_out), n, h,
                                                      _p(pos), _stream(stream)))
    return x_out


def mimo_attn_prefill_swa(cfg: MimoAttnCfg, q, k, v, sinks, out, pos0: int = 0, lse=None, stream=None):
    """q [B,T,Hq,192], k [B,T,Hkv,192], v [B,T,Hkv,128], sinks [Hq] f32 or None, out [B,T,Hq,128]."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, torch.bfloat16, n, 4)
    _need(sinks, torch.float32, "sinks", 1); _need(lse, torch.float32, "lse", 3)
    B, T = q.shape[:2]
    Hq, Hkv = cfg.num_q_heads, cfg.num_kv_heads
    _shape(q, "q", B, T, Hq, 192); _shape(k, "k", B, T, Hkv, 192); _shape(v, "v", B, T, Hkv, 128)
    _shape(out, "out", B, T, Hq, 128); _shape(sinks, "sinks", Hq); _shape(lse, "lse", B, Hq, T)
    _check("mimo_attn_prefill_swa",
           lib.mimo_attn_prefill_swa(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(sinks), B, T, pos0,
                                     _p(out), _p(lse), _stream(stream)))
    return out


def mimo_attn_prefill_workspace_size(cfg: MimoAttnCfg, B: int, total_k: int) -> int:
    return int(load_library().mimo_attn_prefill_workspace_size(ctypes.byref(cfg), B, total_k))


def _prefill_ws(cfg, B, total_k, ws, device):
    """ws: a uint8 device tensor, None (allocate one of the size the call needs) or
    False (no tile images: the attention kernel stages every tile itself)."""
    if ws is False:
        return None, 0
    if ws is None:
        n = mimo_attn_prefill_workspace_size(cfg, B, total_k)
        if n == 0:
            return None, 0
        ws = torch.empty(n, dtype=torch.uint8, device=device)
    return ws, _ws(ws)


def mimo_attn_prefill_global(cfg: MimoAttnCfg, q, k, v, out, q_pos0: int = 0, lse=None, ws=None, stream=None):
    """q [B,Tq,Hq,192] at positions q_pos0.., k/v [B,Tk,Hkv,*] at 0..Tk-1, Tk = q_pos0 + Tq."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, torch.bfloat16, n, 4)
    _need(lse, torch.float32, "lse", 3)
    B, Tq = q.shape[:2]
    Tk = k.shape[1]
    Hq, Hkv = cfg.num_q_heads, cfg.num_kv_heads
    _shape(q, "q", B, Tq, Hq, 192); _shape(k, "k", B, Tk, Hkv, 192); _shape(v, "v", B, Tk, Hkv, 128)
    _shape(out, "out", B, Tq, Hq, 128); _shape(lse, "lse", B, Hq, Tq)
    ws, ws_bytes = _prefill_ws(cfg, B, B * Tk, ws, q.device)
    _check("mimo_attn_prefill_global",
           lib.mimo_attn_prefill_global(ctypes.byref(cfg), _p(q), _p(k), _p(v), B, Tq, Tk, q_pos0,
                                        _p(out), _p(lse), _p(ws), ws_bytes, _stream(stream)))
    return out


def mimo_attn_prefill_varlen(cfg: MimoAttnCfg, q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                             out, k_pos0=None, lse=None, ws=None, stream=None):
    """Packed sequences: q [total_q,Hq,192], k/v [total_k,Hkv,*], out [total_q,Hq,128],
    cu_seqlens_q / cu_seqlens_k [B+1] int32, k_pos0 [B] int64 or None, lse [Hq,total_q]."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, torch.bfloat16, n, 3)
    _need(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1); _need(cu_seqlens_k, torch.int32, "cu_seqlens_k", 1)
    _need(k_pos0, torch.int64, "k_pos0", 1); _need(sinks, torch.float32, "sinks", 1)
    _need(lse, torch.float32, "lse", 2)
    B = cu_seqlens_q.shape[0] - 1
    Hq, Hkv, tq, tk = cfg.num_q_heads, cfg.num_kv_heads, q.shape[0], k.shape[0]
    _shape(q, "q", tq, Hq, 192); _shape(k, "k", tk, Hkv, 192); _shape(v, "v", tk, Hkv, 128)
    _shape(out, "out", tq, Hq, 128); _shape(cu_seqlens_k, "cu_seqlens_k", B + 1); _shape(k_pos0, "k_pos0", B)
    _shape(sinks, "sinks", Hq); _shape(lse, "lse", Hq, tq)
    ws, ws_bytes = _prefill_ws(cfg, B, k.shape[0], ws, q.device)
    _check("mimo_attn_prefill_varlen",
           lib.mimo_attn_prefill_varlen(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(sinks), B, _p(cu_seqlens_q),
                                        _p(cu_seqlens_k), _p(k_pos0), max_seqlen_q, q.shape[0], k.shape[0],
                                        _p(out), _p(lse), _p(ws), ws_bytes, _stream(stream)))
    return out


def mimo_attn_backward_workspace_size(cfg: MimoAttnCfg, B: int, T: int) -> int:
    return int(load_library().mimo_attn_backward_workspace_size(ctypes.byref(cfg), B, T))


def mimo_attn_prefill_backward(cfg: MimoAttnCfg, q, k, v, sinks, out, lse, dout, dq, dk, dv, dsinks=None,
                               pos0: int = 0, ws=None, stream=None):
    """Gradients of a dense prefill: q/dq [B,T,Hq,192], k/dk [B,T,Hkv,192], v/dv [B,T,Hkv,128], out/dout
    [B,T,Hq,128], lse [B,Hq,T] from the forward, dsinks [Hq] (when sinks are given).  ws is allocated
    here when not given."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, torch.bfloat16, n, 4)
    _need(lse, torch.float32, "lse", 3); _need(sinks, torch.float32, "sinks", 1)
    _need(dsinks, torch.float32, "dsinks", 1)
    B, T = q.shape[:2]
    Hq, Hkv = cfg.num_q_heads, cfg.num_kv_heads
    for t, n, h, d in ((q, "q", Hq, 192), (k, "k", Hkv, 192), (v, "v", Hkv, 128), (out, "out", Hq, 128),
                       (dout, "dout", Hq, 128), (dq, "dq", Hq, 192), (dk, "dk", Hkv, 192), (dv, "dv", Hkv, 128)):
        _shape(t, n, B, T, h, d)
    _shape(lse, "lse", B, Hq, T); _shape(sinks, "sinks", Hq); _shape(dsinks, "dsinks", Hq)
    if ws is None:
        ws = torch.empty(max(1, mimo_attn_backward_workspace_size(cfg, B, T)), dtype=torch.uint8, device=q.device)
    ws_bytes = _ws(ws)
    _check("mimo_attn_prefill_backward",
           lib.mimo_attn_prefill_backward(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(sinks), B, T, pos0, _p(out),
                                          _p(lse), _p(dout), _p(dq), _p(dk), _p(dv), _p(dsinks), _p(ws), ws_bytes,
                                          _stream(stream)))
    return dq, dk, dv, dsinks


def _decode_shapes(cfg, S, n_q, cap, q, q_pos, k_cache, v_cache, sinks, out):
    """Shapes of a decode over per-sequence caches (n_q None: one query per sequence)."""
    Hq, Hkv = cfg.num_q_heads, cfg.num_kv_heads
    lead = (S,) if n_q is None else (S, n_q)
    _shape(q, "q", *lead, Hq, 192); _shape(out, "out", *lead, Hq, 128); _shape(q_pos, "q_pos", S)
    _shape(k_cache, "k_cache", S, cap, Hkv, 192); _shape(v_cache, "v_cache", S, cap, Hkv, 128)
    _shape(sinks, "sinks", Hq)


def mimo_attn_decode_workspace_size(cfg: MimoAttnCfg, S: int, cap: int) -> int:
    return int(load_library().mimo_attn_decode_workspace_size(ctypes.byref(cfg), S, cap))


def mimo_attn_decode(cfg: MimoAttnCfg, q, q_pos, k_cache, v_cache, sinks, out, ws=None, stream=None):
    """q [S,Hq,192], q_pos [S] int64, caches [S,cap,Hkv,192|128], out [S,Hq,128].

    ws: a device tensor of at least mimo_attn_decode_workspace_size bytes (any dtype)."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 3); _need(out, torch.bfloat16, "out", 3)
    _need(k_cache, torch.bfloat16, "k_cache", 4); _need(v_cache, torch.bfloat16, "v_cache", 4)
    _need(q_pos, torch.int64, "q_pos", 1); _need(sinks, torch.float32, "sinks", 1)
    S = q.shape[0]
    cap = k_cache.shape[1]
    _decode_shapes(cfg, S, None, cap, q, q_pos, k_cache, v_cache, sinks, out)
    ws_bytes = _ws(ws)
    _check("mimo_attn_decode",
           lib.mimo_attn_decode(ctypes.byref(cfg), S, _p(q), _p(q_pos), _p(k_cache), _p(v_cache), cap,
                                _p(sinks), _p(out), _p(ws), ws_bytes, _stream(stream)))
    return out


def mimo_attn_decode_noalloc(cfg: MimoAttnCfg, q, q_pos, k_cache, v_cache, sinks, out, stream=None):
    """mimo_attn_decode without a workspace: the library's per-GPU scratch holds the
    partials (calls that overlap in time on one GPU race)."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 3); _need(out, torch.bfloat16, "out", 3)
    _need(k_cache, torch.bfloat16, "k_cache", 4); _need(v_cache, torch.bfloat16, "v_cache", 4)
    _need(q_pos, torch.int64, "q_pos", 1); _need(sinks, torch.float32, "sinks", 1)
    S = q.shape[0]
    cap = k_cache.shape[1]
    _decode_shapes(cfg, S, None, cap, q, q_pos, k_cache, v_cache, sinks, out)
    _check("mimo_attn_decode_noalloc",
           lib.mimo_attn_decode_noalloc(ctypes.byref(cfg), S, _p(q), _p(q_pos), _p(k_cache), _p(v_cache), cap,
                                        _p(sinks), _p(out), _stream(stream)))
    return out


def mimo_attn_decode_multi_workspace_size(cfg: MimoAttnCfg, S: int, n_q: int, cap: int) -> int:
    return int(load_library().mimo_attn_decode_multi_workspace_size(ctypes.byref(cfg), S, n_q, cap))


def mimo_attn_decode_multi(cfg: MimoAttnCfg, q, q_pos, k_cache, v_cache, sinks, out, ws=None, stream=None):
    """q [S,n_q,Hq,192], q_pos [S] int64 (newest token), caches [S,cap,Hkv,192|128], out [S,n_q,Hq,128]."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 4); _need(out, torch.bfloat16, "out", 4)
    _need(k_cache, torch.bfloat16, "k_cache", 4); _need(v_cache, torch.bfloat16, "v_cache", 4)
    _need(q_pos, torch.int64, "q_pos", 1); _need(sinks, torch.float32, "sinks", 1)
    S, n_q = q.shape[:2]
    cap = k_cache.shape[1]
    _decode_shapes(cfg, S, n_q, cap, q, q_pos, k_cache, v_cache, sinks, out)
    ws_bytes = _ws(ws)
    _check("mimo_attn_decode_multi",
           lib.mimo_attn_decode_multi(ctypes.byref(cfg), S, n_q, _p(q), _p(q_pos), _p(k_cache), _p(v_cache), cap,
                                      _p(sinks), _p(out), _p(ws), ws_bytes, _stream(stream)))
    return out


KV_DTYPE = {"bf16": 0, "fp8": 1}


def _pool(t, name):
    if t is None or not t.is_cuda or not t.is_contiguous() or t.dim() != 4 or t.dtype not in (torch.bfloat16,
                                                                                            torch.uint8):
        raise ValueError(f"{name} must be a contiguous 4-d CUDA tensor of bfloat16 or uint8 (fp8 codes)")
    return "fp8" if t.dtype == torch.uint8 else "bf16"


def mimo_attn_decode_paged(cfg: MimoAttnCfg, q, q_pos, k_pool, v_pool, block_table, sinks, out, ws=None,
                           k_scale: float = 1.0, v_scale: float = 1.0, stream=None):
    """q [S,n_q,Hq,192], q_pos [S] int64 (newest token), pools [n_blocks,block_size,Hkv,192|128] of bf16 or
    uint8 fp8 e4m3 codes, block_table [S,max_blocks] int32, out [S,n_q,Hq,128]."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 4); _need(out, torch.bfloat16, "out", 4)
    _need(q_pos, torch.int64, "q_pos", 1); _need(sinks, torch.float32, "sinks", 1)
    _need(block_table, torch.int32, "block_table", 2)
    kd, vd = _pool(k_pool, "k_pool"), _pool(v_pool, "v_pool")
    if kd != vd:
        raise ValueError("k_pool and v_pool must have the same element type")
    S, n_q = q.shape[:2]
    n_blocks, block_size = k_pool.shape[:2]
    Hq, Hkv = cfg.num_q_heads, cfg.num_kv_heads
    _shape(q, "q", S, n_q, Hq, 192); _shape(out, "out", S, n_q, Hq, 128); _shape(q_pos, "q_pos", S)
    _shape(k_pool, "k_pool", n_blocks, block_size, Hkv, 192); _shape(v_pool, "v_pool", n_blocks, block_size, Hkv, 128)
    _shape(block_table, "block_table", S, block_table.shape[1]); _shape(sinks, "sinks", Hq)
    ws_bytes = _ws(ws)
    _check("mimo_attn_decode_paged",
           lib.mimo_attn_decode_paged(ctypes.byref(cfg), S, n_q, _p(q), _p(q_pos), _p(k_pool), _p(v_pool), n_blocks,
                                      block_size, KV_DTYPE[kd], k_scale, v_scale, _p(block_table),
                                      block_table.shape[1], _p(sinks), _p(out), _p(ws), ws_bytes, _stream(stream)))
    return out


def mimo_kv_paged_append(cfg: MimoAttnCfg, k_new, v_new, pos, k_pool, v_pool, block_table,
                         k_scale: float = 1.0, v_scale: float = 1.0, stream=None):
    """k_new [S,Hkv,192], v_new [S,Hkv,128] unrotated; writes position pos[s] of each sequence's pages."""
    lib = load_library()
    _need(k_new, torch.bfloat16, "k_new", 3); _need(v_new, torch.bfloat16, "v_new", 3)
    _need(pos, torch.int64, "pos", 1); _need(block_table, torch.int32, "block_table", 2)
    kd, vd = _pool(k_pool, "k_pool"), _pool(v_pool, "v_pool")
    if kd != vd:
        raise ValueError("k_pool and v_pool must have the same element type")
    n_blocks, block_size = k_pool.shape[:2]
    S, Hkv = k_new.shape[0], cfg.num_kv_heads
    _shape(k_new, "k_new", S, Hkv, 192); _shape(v_new, "v_new", S, Hkv, 128); _shape(pos, "pos", S)
    _shape(k_pool, "k_pool", n_blocks, block_size, Hkv, 192); _shape(v_pool, "v_pool", n_blocks, block_size, Hkv, 128)
    _shape(block_table, "block_table", S, block_table.shape[1])
    _check("mimo_kv_paged_append",
           lib.mimo_kv_paged_append(ctypes.byref(cfg), k_new.shape[0], _p(k_new), _p(v_new), _p(pos), _p(k_pool),
                                    _p(v_pool), n_blocks, block_size, KV_DTYPE[kd], k_scale, v_scale,
                                    _p(block_table), block_table.shape[1], _stream(stream)))


def mimo_kv_ring_append(cfg: MimoAttnCfg, k_new, v_new, pos, k_cache, v_cache, stream=None):
    """k_new [S,Hkv,192], v_new [S,Hkv,128] unrotated; writes slot pos mod cap of the caches."""
    lib = load_library()
    _need(k_new, torch.bfloat16, "k_new", 3); _need(v_new, torch.bfloat16, "v_new", 3)
    _need(k_cache, torch.bfloat16, "k_cache", 4); _need(v_cache, torch.bfloat16, "v_cache", 4)
    _need(pos, torch.int64, "pos", 1)
    S = k_new.shape[0]
    cap = k_cache.shape[1]
    Hkv = cfg.num_kv_heads
    _shape(k_new, "k_new", S, Hkv, 192); _shape(v_new, "v_new", S, Hkv, 128); _shape(pos, "pos", S)
    _shape(k_cache, "k_cache", S, cap, Hkv, 192); _shape(v_cache, "v_cache", S, cap, Hkv, 128)
    _check("mimo_kv_ring_append",
           lib.mimo_kv_ring_append(ctypes.byref(cfg), S, _p(k_new), _p(v_new), _p(pos), _p(k_cache),
                                   _p(v_cache), cap, _stream(stream)))
    return k_cache, v_cache


# ---------------------------------------------------------------- on-box peaks (libmimo_peaks.so)
# Measurement only: the benchmark reports the attention kernels against what
# these loops reach on the same card, next to the vendor peaks.

PEAKS_PATH = os.path.join(_PKG, "libmimo_peaks.so")
_peaks = None


def load_peaks(path: str = PEAKS_PATH):
    global _peaks
    if _peaks is not None:
        return _peaks
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with global_attention_sinks_amd.build.build()")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.mimo_peak_mfma_waves.argtypes = []
    lib.mimo_peak_mfma_bf16.argtypes = [P, I64, I32, P, P]
    lib.mimo_peak_copy.argtypes = [P, P, I64, P]
    lib.mimo_peak_read.argtypes = [P, I64, P, P]
    lib.mimo_peak_write.argtypes = [P, I64, ctypes.c_uint32, P]
    for fn in ("mimo_peak_mfma_waves", "mimo_peak_mfma_bf16", "mimo_peak_copy", "mimo_peak_read", "mimo_peak_write"):
        getattr(lib, fn).restype = ctypes.c_int
    _peaks = lib
    return lib


def _hip_ok(fn: str, err: int):
    if err != 0:
        raise RuntimeError(f"{fn}: hipError {err}")


def peak_mfma_flops(iters: int) -> int:
    """FLOP of one mimo_peak_mfma_bf16 launch."""
    return int(load_peaks().mimo_peak_mfma_waves()) * iters * 64 * 32768


def peak_mfma_bf16(operands, iters: int, sink, stream=None):
    """operands: bf16 CUDA tensor (>= 64 values); sink: float32 CUDA tensor of
    mimo_peak_mfma_waves() values."""
    lib = load_peaks()
    _need(operands, torch.bfloat16, "operands")
    _need(sink, torch.float32, "sink")
    if sink.numel() < lib.mimo_peak_mfma_waves() or operands.numel() < 64:
        raise ValueError("sink needs mimo_peak_mfma_waves() floats and operands >= 64 values")
    _hip_ok("mimo_peak_mfma_bf16", lib.mimo_peak_mfma_bf16(_p(operands), operands.numel(), iters, _p(sink),
                                                           _stream(stream)))


def peak_copy(src, dst, stream=None):
    lib = load_peaks()
    n = src.numel() * src.element_size()
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()) or \
            dst.numel() * dst.element_size() < n:
        raise ValueError("src and dst must be contiguous CUDA tensors, dst at least as large")
    _hip_ok("mimo_peak_copy", lib.mimo_peak_copy(_p(src), _p(dst), n, _stream(stream)))


def peak_read(src, out, stream=None):
    lib = load_peaks()
    if not (src.is_cuda and src.is_contiguous() and out.is_cuda):
        raise ValueError("src and out must be CUDA tensors")
    _hip_ok("mimo_peak_read", lib.mimo_peak_read(_p(src), src.numel() * src.element_size(), _p(out),
                                                 _stream(stream)))


def peak_write(dst, value: int = 0, stream=None):
    lib = load_peaks()
    if not (dst.is_cuda and dst.is_contiguous()):
        raise ValueError("dst must be a contiguous CUDA tensor")
    _hip_ok("mimo_peak_write", lib.mimo_peak_write(_p(dst), dst.numel() * dst.element_size(), value,
                                                   _stream(stream)))
