"""Seeded synthetic inputs for the MiMo-V2.6-Flash attention hot path.

This module holds no attention arithmetic: only random draws, bf16 rounding of
those draws, and the shapes of the workloads.  Both the fp64 oracle (tests and
the CPU baseline) and the HIP path are fed from here, so neither side ever
produces the other's inputs.

Recipe (every workload):
  * root = numpy SeedSequence(seed); its first five spawned children seed, in
    order, q, k, v, the sink logits and the positions / lengths.
  * each tensor is drawn in fixed blocks of BLOCK elements; block b uses the
    b-th spawned child of the tensor's seed, so the values do not depend on how
    many threads fill them.
  * normal draws are float32 N(0, 1), rounded to bf16 by round-to-nearest-even;
    sinks stay float32 N(0, 1).
  * cache slots that hold no token are filled with a bf16 quiet NaN (0x7FC0) so
    that any read of them shows up in the output.

Arrays of bf16 values are numpy uint16 holding the bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK = 1 << 24
BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bits.

    Finite inputs only (normal draws are always finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(seed: np.random.SeedSequence, shape) -> np.ndarray:
    """float32 N(0,1) draws rounded to bf16, filled block by block."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nblk = max(1, math.ceil(n / BLOCK))
    kids = seed.spawn(nblk)

    def fill(b):
        lo, hi = b * BLOCK, min(n, (b + 1) * BLOCK)
        rng = np.random.Generator(np.random.PCG64(kids[b]))
        out[lo:hi] = f32_to_bf16_bits(rng.standard_normal(hi - lo, dtype=np.float32))

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def normal_bf16_slice(seed: np.random.SeedSequence, shape, lo: int, hi: int) -> np.ndarray:
    """Elements [lo, hi) of the flattened normal_bf16(seed, shape), drawing only
    the blocks that cover them."""
    n = int(np.prod(shape))
    assert 0 <= lo <= hi <= n
    nblk = max(1, math.ceil(n / BLOCK))
    kids = seed.spawn(nblk)
    b0, b1 = lo // BLOCK, (hi + BLOCK - 1) // BLOCK
    out = np.empty(hi - lo, dtype=np.uint16)

    def fill(b):
        blo, bhi = b * BLOCK, min(n, (b + 1) * BLOCK)
        rng = np.random.Generator(np.random.PCG64(kids[b]))
        vals = f32_to_bf16_bits(rng.standard_normal(bhi - blo, dtype=np.float32))
        s0, s1 = max(lo, blo), min(hi, bhi)
        out[s0 - lo:s1 - lo] = vals[s0 - blo:s1 - blo]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(b0, b1)))
    return out


def normal_f32(seed: np.random.SeedSequence, shape) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)


def children(seed: int):
    """The five child seeds of a workload: q, k, v, sinks, positions."""
    return np.random.SeedSequence(seed).spawn(5)


_children = children


# Head layout of the two layer types (model facts, not method arithmetic).
SWA_HEADS = (64, 8)
GLOBAL_HEADS = (64, 4)
D_QK, D_V = 192, 128


def prefill_inputs(B: int, T: int, n_q_heads: int, n_kv_heads: int, seed: int,
                   with_sinks: bool, Tk: int | None = None) -> dict:
    """q [B,T,Hq,192], k/v [B,Tk,Hkv,192|128] bf16 bits; sinks [Hq] f32 or None.

    Tk defaults to T (keys are the same tokens as the queries)."""
    Tk = T if Tk is None else Tk
    cq, ck, cv, cs, _ = _children(seed)
    return {
        "q": normal_bf16(cq, (B, T, n_q_heads, D_QK)),
        "k": normal_bf16(ck, (B, Tk, n_kv_heads, D_QK)),
        "v": normal_bf16(cv, (B, Tk, n_kv_heads, D_V)),
        "sinks": normal_f32(cs, (n_q_heads,)) if with_sinks else None,
    }


def decode_inputs(S: int, cap: int, n_q_heads: int, n_kv_heads: int, seed: int,
                  window: int, pos_lo: int, pos_hi: int, with_sinks: bool,
                  poison: bool = True) -> dict:
    """One query token per sequence over a KV cache [S,cap,Hkv,D].

    window > 0 (sliding layer): positions p ~ U[pos_lo, pos_hi) (half-open);
    the cache is a ring and every slot whose token lies in the window
    [p-window+1, p] holds a draw.
    window == 0 (global layer): KV lengths L ~ U[pos_lo, pos_hi] (closed),
    p = L-1, slots 0..L-1 hold draws.
    All other slots hold bf16 NaN when poison is set, else draws too.
    The cache holds post-RoPE keys and plain values."""
    cq, ck, cv, cs, cp = _children(seed)
    rng = np.random.Generator(np.random.PCG64(cp))
    if window > 0:
        pos = rng.integers(pos_lo, pos_hi, size=S, dtype=np.int64)
    else:
        pos = rng.integers(pos_lo, pos_hi, size=S, dtype=np.int64, endpoint=True) - 1
    q = normal_bf16(cq, (S, n_q_heads, D_QK))
    kc = np.empty((S, cap, n_kv_heads, D_QK), dtype=np.uint16)
    vc = np.empty((S, cap, n_kv_heads, D_V), dtype=np.uint16)
    kseeds = ck.spawn(S)
    vseeds = cv.spawn(S)
    for s in range(S):
        p = int(pos[s])
        if window > 0:
            live = np.zeros(cap, dtype=bool)
            lo = max(0, p - window + 1)
            live[np.arange(lo, p + 1) % cap] = True
        else:
            live = np.arange(cap) <= p
        n_live = int(live.sum())
        kvals = normal_bf16(kseeds[s], (n_live, n_kv_heads, D_QK))
        vvals = normal_bf16(vseeds[s], (n_live, n_kv_heads, D_V))
        fill = BF16_NAN if poison else np.uint16(0)
        kc[s] = fill
        vc[s] = fill
        kc[s][live] = kvals
        vc[s][live] = vvals
    return {
        "q": q, "pos": pos, "k_cache": kc, "v_cache": vc,
        "sinks": normal_f32(cs, (n_q_heads,)) if with_sinks else None,
    }


def decode_multi_inputs(S: int, n_q: int, cap: int, n_q_heads: int, n_kv_heads: int, seed: int,
                        window: int, pos: np.ndarray, with_sinks: bool) -> dict:
    """n_q query tokens per sequence [S,n_q,Hq,192], the newest at pos[s], over a
    cache [S,cap,Hkv,D] in which the slots of the positions some token can see
    (pos - n_q + 1 - window + 1 .. pos for a ring, 0 .. pos otherwise) hold draws
    and every other slot holds bf16 NaN."""
    cq, ck, cv, cs, _ = _children(seed)
    pos = np.asarray(pos, dtype=np.int64)
    q = normal_bf16(cq, (S, n_q, n_q_heads, D_QK))
    kc = np.full((S, cap, n_kv_heads, D_QK), BF16_NAN, dtype=np.uint16)
    vc = np.full((S, cap, n_kv_heads, D_V), BF16_NAN, dtype=np.uint16)
    kseeds, vseeds = ck.spawn(S), cv.spawn(S)
    for s in range(S):
        p = int(pos[s])
        if p < 0:
            continue
        lo = max(0, p - (n_q - 1) - window + 1) if window > 0 else 0
        slots = np.arange(lo, p + 1) % cap
        kc[s, slots] = normal_bf16(kseeds[s], (len(slots), n_kv_heads, D_QK))
        vc[s, slots] = normal_bf16(vseeds[s], (len(slots), n_kv_heads, D_V))
    return {"q": q, "pos": pos, "k_cache": kc, "v_cache": vc,
            "sinks": normal_f32(cs, (n_q_heads,)) if with_sinks else None}


FP8_NAN = np.uint8(0x7F)


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 draws to OCP fp8 e4m3 codes (round to nearest even, via
    torch's float8_e4m3fn cast), after clipping them to the format's +-448."""
    import torch
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def paged_decode_inputs(S: int, n_q: int, block_size: int, n_q_heads: int, n_kv_heads: int, seed: int,
                        window: int, pos: np.ndarray, with_sinks: bool, kv_dtype: str = "bf16",
                        k_scale: float = 1.0, v_scale: float = 1.0, spare_blocks: int = 3) -> dict:
    """n_q query tokens per sequence (newest at pos[s]) over a paged cache.

    Sequence s holds positions 0..pos[s] in blocks of block_size slots; with a
    window only the blocks that hold some token's window get a pool block (the
    table entry of the others is -1).  Pool blocks are handed out in a seeded
    random order, plus spare_blocks unused ones.  Slots of the positions some
    token can see hold draws: bf16 N(0,1), or fp8 e4m3 codes of N(0,1) / scale;
    every other slot holds NaN (bf16 0x7FC0, fp8 0x7F)."""
    cq, ck, cv, cs, cp = _children(seed)
    pos = np.asarray(pos, dtype=np.int64)
    fp8 = kv_dtype == "fp8"
    q = normal_bf16(cq, (S, n_q, n_q_heads, D_QK))
    max_blocks = int(max(1, max((int(p) + block_size) // block_size for p in pos))) + 1
    table = np.full((S, max_blocks), -1, dtype=np.int32)
    need = []
    for s in range(S):
        p = int(pos[s])
        if p < 0:
            continue
        lo = max(0, p - (n_q - 1) - window + 1) if window > 0 else 0
        for b in range(lo // block_size, p // block_size + 1):
            need.append((s, b))
    n_blocks = len(need) + spare_blocks
    perm = np.random.Generator(np.random.PCG64(cp)).permutation(n_blocks)
    for i, (s, b) in enumerate(need):
        table[s, b] = perm[i]
    nan = FP8_NAN if fp8 else BF16_NAN
    dt = np.uint8 if fp8 else np.uint16
    kp = np.full((n_blocks, block_size, n_kv_heads, D_QK), nan, dtype=dt)
    vp = np.full((n_blocks, block_size, n_kv_heads, D_V), nan, dtype=dt)
    kseeds, vseeds = ck.spawn(S), cv.spawn(S)
    for s in range(S):
        p = int(pos[s])
        if p < 0:
            continue
        lo = max(0, p - (n_q - 1) - window + 1) if window > 0 else 0
        tpos = np.arange(lo, p + 1)
        blk = table[s, tpos // block_size]
        slot = tpos % block_size
        if fp8:
            kd = np.random.Generator(np.random.PCG64(kseeds[s])).standard_normal(
                (len(tpos), n_kv_heads, D_QK), dtype=np.float32)
            vd = np.random.Generator(np.random.PCG64(vseeds[s])).standard_normal(
                (len(tpos), n_kv_heads, D_V), dtype=np.float32)
            kp[blk, slot] = f32_to_e4m3_codes(kd / np.float32(k_scale))
            vp[blk, slot] = f32_to_e4m3_codes(vd / np.float32(v_scale))
        else:
            kp[blk, slot] = normal_bf16(kseeds[s], (len(tpos), n_kv_heads, D_QK))
            vp[blk, slot] = normal_bf16(vseeds[s], (len(tpos), n_kv_heads, D_V))
    return {"q": q, "pos": pos, "k_pool": kp, "v_pool": vp, "table": table, "block_size": block_size,
            "kv_dtype": kv_dtype, "k_scale": float(k_scale), "v_scale": float(v_scale),
            "sinks": normal_f32(cs, (n_q_heads,)) if with_sinks else None}


def global_prefill_chunk(T: int, n_q_heads: int, n_kv_heads: int, seed: int, t_lo: int, t_hi: int,
                         kv: bool = True) -> dict:
    """Query rows [t_lo, t_hi) of a B=1 prefill of T tokens and (kv=True) the
    keys/values 0..t_hi-1, drawn exactly as prefill_inputs(1, T, ...) would draw them."""
    cq, ck, cv, _, _ = children(seed)
    row_q, row_k, row_v = n_q_heads * D_QK, n_kv_heads * D_QK, n_kv_heads * D_V
    q = normal_bf16_slice(cq, (1, T, n_q_heads, D_QK), t_lo * row_q, t_hi * row_q)
    out = {"q": q.reshape(1, t_hi - t_lo, n_q_heads, D_QK)}
    if kv:
        k = normal_bf16_slice(ck, (1, T, n_kv_heads, D_QK), 0, t_hi * row_k)
        v = normal_bf16_slice(cv, (1, T, n_kv_heads, D_V), 0, t_hi * row_v)
        out["k"] = k.reshape(1, t_hi, n_kv_heads, D_QK)
        out["v"] = v.reshape(1, t_hi, n_kv_heads, D_V)
    return out


def varlen_inputs(lens_q, lens_k, n_q_heads: int, n_kv_heads: int, seed: int, with_sinks: bool,
                  k_pos0=None) -> dict:
    """Packed (THD) sequences: sequence b has lens_q[b] query tokens and
    lens_k[b] key tokens, stored back to back.  q [sum(lens_q),Hq,192],
    k/v [sum(lens_k),Hkv,*] bf16 bits; cu_q / cu_k [B+1] int32 offsets;
    k_pos0 [B] int64 (position of each sequence's first key) or None."""
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_k = np.asarray(lens_k, dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    cq, ck, cv, cs, _ = _children(seed)
    return {
        "q": normal_bf16(cq, (int(cu_q[-1]), n_q_heads, D_QK)),
        "k": normal_bf16(ck, (int(cu_k[-1]), n_kv_heads, D_QK)),
        "v": normal_bf16(cv, (int(cu_k[-1]), n_kv_heads, D_V)),
        "cu_q": cu_q, "cu_k": cu_k,
        "k_pos0": None if k_pos0 is None else np.asarray(k_pos0, dtype=np.int64),
        "sinks": normal_f32(cs, (n_q_heads,)) if with_sinks else None,
    }


def append_inputs(S: int, n_kv_heads: int, seed: int, pos_lo: int, pos_hi: int) -> dict:
    """New-token k/v rows [S,Hkv,192|128] and their positions ~ U[pos_lo,pos_hi)."""
    cq, ck, cv, cs, cp = _children(seed)
    rng = np.random.Generator(np.random.PCG64(cp))
    return {
        "k": normal_bf16(ck, (S, n_kv_heads, D_QK)),
        "v": normal_bf16(cv, (S, n_kv_heads, D_V)),
        "pos": rng.integers(pos_lo, pos_hi, size=S, dtype=np.int64),
    }


def rope_inputs(n_tokens: int, n_heads: int, seed: int, pos_lo: int, pos_hi: int) -> dict:
    cq, ck, cv, cs, cp = _children(seed)
    rng = np.random.Generator(np.random.PCG64(cp))
    return {
        "x": normal_bf16(cq, (n_tokens, n_heads, D_QK)),
        "pos": rng.integers(pos_lo, pos_hi, size=n_tokens, dtype=np.int64),
    }


# The five workloads, by what they are.  Seeds are 1000 + index.
WORKLOADS = {
    "swa_prefill_t512": dict(kind="swa_prefill", B=1, T=512, seed=1000),
    "swa_prefill_b4_t8192": dict(kind="swa_prefill", B=4, T=8192, seed=1001),
    "global_prefill_t32768": dict(kind="global_prefill", B=1, T=32768, seed=1002),
    "mixed_decode_64swa_16global": dict(kind="mixed_decode", S_swa=64, S_global=16,
                                        swa_cap=128, global_cap=131072, seed=1003),
    "global_prefill_t524288_chunked": dict(kind="global_prefill", B=1, T=524288,
                                           chunk=65536, seed=1004),
}
