"""fp64 CPU oracle for the MiMo-V2.6-Flash attention hot path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use it; the product path never imports it.  It shares no code
with the HIP library (see mimo_oracle.c for what is computed and where each
step is stated on the pages).

Every function takes numpy arrays (bf16 as uint16 bit patterns, positions as
int64) and returns fp64 arrays.  Layouts follow the library's: token-major
[tokens, heads, dim].

Parity status: partial RoPE's pairing (rotate-half, not interleaved) and its
frequency exponent over rope_dim are readings of the pages (they print the
[rope, nope] split and the default rope type, not the rotation itself); the
invariants in the tests hold for either pairing, so that one convention is
"parity unpinned" by the pages.  Everything else is pinned by the tests in
tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mimo_oracle.c")
_LIB = os.path.join(_HERE, "libmimo_oracle.so")

ROPE_DIM = 64
SOFTMAX_SCALE = 1.0 / math.sqrt(192.0)
V_SCALE = 0.707
SWA_WINDOW = 128
SWA_BASE = 1.0e4
GLOBAL_BASE = 1.0e7


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math) and OpenMP."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-Wall", "-Werror", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=not os.path.exists(_LIB))
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.oracle_rope_partial.argtypes = [P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, P, ctypes.c_double, P]
        lib.oracle_rope_partial.restype = None
        lib.oracle_attention.argtypes = [
            P, P, ctypes.c_int64, P, ctypes.c_int, P, ctypes.c_int64, P,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, P, ctypes.c_int64, ctypes.c_double, ctypes.c_double,
            P, P, P, ctypes.c_int]
        lib.oracle_attention.restype = None
        lib.oracle_attention_backward.argtypes = [
            P, P, ctypes.c_int64, P, P, ctypes.c_int64, P,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, P, ctypes.c_int64, ctypes.c_double, ctypes.c_double,
            P, P, P, P, P, ctypes.c_int]
        lib.oracle_attention_backward.restype = None
        lib.oracle_operand_rounding.argtypes = [
            P, P, ctypes.c_int64, P, P, ctypes.c_int64, P,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, P, ctypes.c_int64, ctypes.c_double, ctypes.c_double, P, P, ctypes.c_int]
        lib.oracle_operand_rounding.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def rope_partial(x: np.ndarray, pos: np.ndarray, base: float, rope_dim: int = ROPE_DIM) -> np.ndarray:
    """x [n_tok, n_heads, D] bf16 bits, pos [n_tok] -> rotated fp64 [n_tok, n_heads, D]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    n, h, d = x.shape
    out = np.empty((n, h, d), dtype=np.float64)
    _load().oracle_rope_partial(_ptr(x), n, h, d, rope_dim, _ptr(pos), float(base), _ptr(out))
    return out


def attention(q, q_pos, k, k_pos, v, *, sinks=None, window: int = 0, base: float,
              k_rotated: bool = False, softmax_scale: float = SOFTMAX_SCALE,
              v_scale: float = V_SCALE, rope_dim: int = ROPE_DIM,
              want_lse: bool = False, want_psink: bool = False, n_threads: int = 0):
    """Rows of one sequence.  q [nq,Hq,Dqk], k [nk,Hkv,Dqk], v [nk,Hkv,Dv] bf16 bits.

    Returns out [nq,Hq,Dv] fp64, plus lse / psink [nq,Hq] when asked."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    k_pos = np.ascontiguousarray(k_pos, dtype=np.int64)
    nq, hq, dqk = q.shape
    nk, hkv, _ = k.shape
    dv = v.shape[2]
    assert hq % hkv == 0 and k.shape[2] == dqk and v.shape[:2] == (nk, hkv)
    assert q_pos.shape == (nq,) and k_pos.shape == (nk,)
    s = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float64)
    out = np.empty((nq, hq, dv), dtype=np.float64)
    lse = np.empty((nq, hq), dtype=np.float64) if want_lse else None
    psink = np.empty((nq, hq), dtype=np.float64) if want_psink else None
    _load().oracle_attention(_ptr(q), _ptr(q_pos), nq, _ptr(k), int(k_rotated), _ptr(k_pos), nk,
                             _ptr(v), hq, hkv, dqk, dv, rope_dim, float(base), _ptr(s),
                             int(window), float(softmax_scale), float(v_scale),
                             _ptr(out), _ptr(lse), _ptr(psink), int(n_threads))
    res = [out]
    if want_lse:
        res.append(lse)
    if want_psink:
        res.append(psink)
    return res[0] if len(res) == 1 else tuple(res)


def attention_backward(q, q_pos, k, k_pos, v, dout, *, sinks=None, window: int = 0, base: float,
                       softmax_scale: float = SOFTMAX_SCALE, v_scale: float = V_SCALE,
                       rope_dim: int = ROPE_DIM, n_threads: int = 0):
    """Gradients of attention() for one sequence (k unrotated): returns dq [nq,Hq,Dqk],
    dk [nk,Hkv,Dqk], dv [nk,Hkv,Dv] and dsinks [Hq] (None without sinks), fp64."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    dout = np.ascontiguousarray(dout, dtype=np.uint16)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    k_pos = np.ascontiguousarray(k_pos, dtype=np.int64)
    nq, hq, dqk = q.shape
    nk, hkv, _ = k.shape
    dv_ = v.shape[2]
    assert dout.shape == (nq, hq, dv_)
    s = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float64)
    dq = np.empty((nq, hq, dqk))
    dk = np.empty((nk, hkv, dqk))
    dv = np.empty((nk, hkv, dv_))
    ds = np.empty(hq) if sinks is not None else None
    _load().oracle_attention_backward(_ptr(q), _ptr(q_pos), nq, _ptr(k), _ptr(k_pos), nk, _ptr(v), hq, hkv, dqk,
                                      dv_, rope_dim, float(base), _ptr(s), int(window), float(softmax_scale),
                                      float(v_scale), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ds),
                                      int(n_threads))
    return dq, dk, dv, ds


def operand_rounding(q, q_pos, k, k_pos, v, *, sinks=None, window: int = 0, base: float,
                     softmax_scale: float = SOFTMAX_SCALE, v_scale: float = V_SCALE,
                     rope_dim: int = ROPE_DIM, n_threads: int = 0):
    """What holding rope(q) and rope(k) as bf16 operands does to attention() (k
    unrotated): returns (out_rounded, bound), both [nq,Hq,Dv] fp64 --
    out_rounded: the rows with the rotated dims of rope(q) and rope(k_j) rounded
    to the nearest bf16 before the scores; bound: the largest change of the exact
    rows that any rounding within bf16's unit roundoff 2^-8 can cause (derived in
    mimo_oracle.c, no first-order approximation)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    k_pos = np.ascontiguousarray(k_pos, dtype=np.int64)
    nq, hq, dqk = q.shape
    nk, hkv, _ = k.shape
    dv = v.shape[2]
    s = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float64)
    out_r = np.empty((nq, hq, dv))
    bound = np.empty((nq, hq, dv))
    _load().oracle_operand_rounding(_ptr(q), _ptr(q_pos), nq, _ptr(k), _ptr(k_pos), nk, _ptr(v), hq, hkv, dqk,
                                    dv, rope_dim, float(base), _ptr(s), int(window), float(softmax_scale),
                                    float(v_scale), _ptr(out_r), _ptr(bound), int(n_threads))
    return out_r, bound


def prefill_backward(q, k, v, dout, *, sinks=None, pos0: int = 0, window: int, base: float, n_threads: int = 0):
    """Gradients of a dense prefill batch (q [B,T,Hq,192], k/v [B,T,Hkv,*], token t at
    pos0 + t, dout [B,T,Hq,128]): dq, dk, dv per batch entry and dsinks summed over
    the batch."""
    B, T = q.shape[:2]
    pos = pos0 + np.arange(T, dtype=np.int64)
    outs = [attention_backward(q[b], pos, k[b], pos, v[b], dout[b], sinks=sinks, window=window, base=base,
                               n_threads=n_threads) for b in range(B)]
    dq = np.stack([o[0] for o in outs])
    dk = np.stack([o[1] for o in outs])
    dv = np.stack([o[2] for o in outs])
    ds = None if sinks is None else np.sum([o[3] for o in outs], axis=0)
    return dq, dk, dv, ds


def prefill_swa(q, k, v, sinks, *, pos0: int = 0, window: int = SWA_WINDOW, base: float = SWA_BASE,
                rows=None, want_lse: bool = False, n_threads: int = 0):
    """Sliding-window prefill of a batch: q [B,T,Hq,192], k/v [B,T,Hkv,*], token t at pos0+t.

    rows: optional array of token indices to evaluate (same for every batch entry).
    Returns out [B,len(rows),Hq,128] (and lse [B,len(rows),Hq])."""
    B, T = q.shape[:2]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    kpos = pos0 + np.arange(T, dtype=np.int64)
    outs, lses = [], []
    for b in range(B):
        # keys that any selected row can see: [min(rows)-window+1, max(rows)]
        lo = max(0, int(rows.min()) - window + 1) if len(rows) else 0
        hi = int(rows.max()) + 1 if len(rows) else 0
        r = attention(q[b, rows], pos0 + rows, k[b, lo:hi], kpos[lo:hi], v[b, lo:hi],
                      sinks=sinks, window=window, base=base, want_lse=want_lse, n_threads=n_threads)
        if want_lse:
            outs.append(r[0]); lses.append(r[1])
        else:
            outs.append(r)
    out = np.stack(outs)
    return (out, np.stack(lses)) if want_lse else out


def prefill_global(q, k, v, *, q_pos0: int = 0, base: float = GLOBAL_BASE, rows=None,
                   want_lse: bool = False, n_threads: int = 0):
    """Causal prefill: q [B,Tq,Hq,192] at positions q_pos0.., k/v [B,Tk,Hkv,*] at 0..Tk-1."""
    B, Tq = q.shape[:2]
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    hi = q_pos0 + (int(rows.max()) + 1 if len(rows) else 0)
    kpos = np.arange(hi, dtype=np.int64)
    outs, lses = [], []
    for b in range(B):
        r = attention(q[b, rows], q_pos0 + rows, k[b, :hi], kpos, v[b, :hi],
                      window=0, base=base, want_lse=want_lse, n_threads=n_threads)
        if want_lse:
            outs.append(r[0]); lses.append(r[1])
        else:
            outs.append(r)
    out = np.stack(outs)
    return (out, np.stack(lses)) if want_lse else out


def prefill_varlen(q, k, v, cu_q, cu_k, *, k_pos0=None, sinks=None, window: int, base: float,
                   want_lse: bool = False, n_threads: int = 0):
    """Packed sequences: sequence b owns query tokens cu_q[b]..cu_q[b+1]-1 and key
    tokens cu_k[b]..cu_k[b+1]-1; its first key sits at position k_pos0[b] (0 if
    None) and its queries are its last keys (query t at k_pos0[b] + Tk - Tq + t).

    Returns out [total_q,Hq,128] (and lse [Hq,total_q]); rows outside every
    sequence are NaN."""
    total_q, hq = q.shape[:2]
    out = np.full((total_q, hq, v.shape[2]), np.nan)
    lse = np.full((hq, total_q), np.nan)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if qe == qs:
            continue
        p0 = 0 if k_pos0 is None else int(k_pos0[b])
        kpos = p0 + np.arange(ke - ks, dtype=np.int64)
        qpos = kpos[ke - ks - (qe - qs):]
        r = attention(q[qs:qe], qpos, k[ks:ke], kpos, v[ks:ke], sinks=sinks, window=window, base=base,
                      want_lse=want_lse, n_threads=n_threads)
        if want_lse:
            out[qs:qe], lse[:, qs:qe] = r[0], r[1].T
        else:
            out[qs:qe] = r
    return (out, lse) if want_lse else out


def cache_slots(p: int, cap: int, window: int):
    """Cache rule: the token at position t lives in slot t mod cap.  A query at
    position p sees positions max(0, p-window+1)..p (window > 0) or 0..p."""
    lo = max(0, p - window + 1) if window > 0 else 0
    tpos = np.arange(lo, p + 1, dtype=np.int64)
    return tpos % cap, tpos


def decode(q, q_pos, k_cache, v_cache, *, sinks=None, window: int, base: float,
           seqs=None, n_threads: int = 0):
    """One query per sequence over a post-RoPE KV cache [S,cap,Hkv,*].

    q [S,Hq,192] unrotated.  Returns out [len(seqs),Hq,128] fp64."""
    S = q.shape[0]
    cap = k_cache.shape[1]
    seqs = range(S) if seqs is None else seqs
    outs = []
    for s in seqs:
        p = int(q_pos[s])
        slots, tpos = cache_slots(p, cap, window)
        outs.append(attention(q[s:s + 1], np.array([p]), k_cache[s, slots], tpos, v_cache[s, slots],
                              sinks=sinks, window=window, base=base, k_rotated=True,
                              n_threads=n_threads)[0])
    return np.stack(outs)


def decode_multi(q, q_pos, k_cache, v_cache, *, sinks=None, window: int, base: float, seqs=None,
                 n_threads: int = 0):
    """n_q query tokens per sequence, the newest at q_pos[s], token i at
    q_pos[s] - (n_q - 1 - i); each sees the cache tokens its own position sees.
    q [S,n_q,Hq,192] unrotated.  Returns out [len(seqs),n_q,Hq,128] fp64
    (a token at a negative position gets zeros)."""
    S, nq, hq = q.shape[:3]
    cap = k_cache.shape[1]
    seqs = range(S) if seqs is None else seqs
    outs = np.zeros((len(seqs), nq, hq, v_cache.shape[3]))
    for r, s in enumerate(seqs):
        for i in range(nq):
            p = int(q_pos[s]) - (nq - 1 - i)
            if p < 0:
                continue
            slots, tpos = cache_slots(p, cap, window)
            outs[r, i] = attention(q[s, i][None], np.array([p]), k_cache[s, slots], tpos, v_cache[s, slots],
                                   sinks=sinks, window=window, base=base, k_rotated=True, n_threads=n_threads)[0]
    return outs


# ---------------------------------------------------------------- fp8 e4m3 (OCP) and paged caches

def e4m3_to_f64(codes) -> np.ndarray:
    """OCP fp8 e4m3 (e4m3fn) codes to their values: sign bit 7, exponent bits 6..3
    with bias 7, mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); the
    all-ones exponent with all-ones mantissa is NaN (no infinities)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


_E4M3_POS = None


def e4m3_round(x) -> np.ndarray:
    """Values to e4m3 codes: nearest representable value, ties to the even code
    (the one with an even mantissa), magnitudes beyond 448 saturated to 448."""
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = e4m3_to_f64(np.arange(0x7F))          # codes 0..126: 0 .. 448, increasing
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == _E4M3_POS[hi], hi, pick)
    return (pick | np.where(x < 0, 0x80, 0)).astype(np.uint8)


def _bf16_bits_exact(x: np.ndarray) -> np.ndarray:
    """fp64 values that bf16 represents exactly, as bf16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(x, np.float64), equal_nan=True)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def decode_paged(q, q_pos, k_pool, v_pool, table, *, block_size: int, kv_dtype: str = "bf16",
                 k_scale: float = 1.0, v_scale: float = 1.0, sinks=None, window: int, base: float,
                 seqs=None, n_threads: int = 0):
    """decode_multi over a paged cache: position t of sequence s sits in pool
    block table[s, t // block_size], slot t % block_size.  fp8 pools hold e4m3
    codes of value code * scale: the codes' values are exact in bf16, and the
    scales multiply the scores (k) and the output (v)."""
    S, nq, hq = q.shape[:3]
    seqs = range(S) if seqs is None else seqs
    outs = np.zeros((len(seqs), nq, hq, v_pool.shape[3]))
    fp8 = kv_dtype == "fp8"
    for r, s in enumerate(seqs):
        for i in range(nq):
            p = int(q_pos[s]) - (nq - 1 - i)
            if p < 0:
                continue
            tpos = np.arange(max(0, p - window + 1) if window > 0 else 0, p + 1, dtype=np.int64)
            blk = table[s, tpos // block_size]
            assert np.all(blk >= 0)
            kr, vr = k_pool[blk, tpos % block_size], v_pool[blk, tpos % block_size]
            if fp8:
                kr, vr = _bf16_bits_exact(e4m3_to_f64(kr)), _bf16_bits_exact(e4m3_to_f64(vr))
            outs[r, i] = attention(q[s, i][None], np.array([p]), kr, tpos, vr, sinks=sinks, window=window,
                                   base=base, k_rotated=True, n_threads=n_threads,
                                   softmax_scale=SOFTMAX_SCALE * (k_scale if fp8 else 1.0),
                                   v_scale=V_SCALE * (v_scale if fp8 else 1.0))[0]
    return outs


def kv_paged_append_fp8(k_new, v_new, pos, base: float, k_scale: float, v_scale: float):
    """What an fp8 paged append stores: codes of rope(k_new at pos) / k_scale and
    of v_new / v_scale, each rounded once from its fp64 value."""
    kr = rope_partial(k_new, pos, base)
    v = bf16_to_f64(v_new)
    return e4m3_round(kr / k_scale), e4m3_round(v / v_scale), kr / k_scale, v / v_scale


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns to their fp64 values."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def kv_ring_append_rows(k_new, v_new, pos, base: float):
    """What the append writes: rope(k_new) at pos and v_new unchanged, fp64."""
    return rope_partial(k_new, pos, base), v_new
