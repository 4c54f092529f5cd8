"""GPU parity on shapes drawn from a fixed seed: irregular batch sizes, lengths, windows,
positions, head groupings and workspace choices for the prefill, decode and backward
calls, each compared element by element with the fp64 oracle (the same bar as the
hand-picked cases).  The draw happens once at import, so the cases are the same on
every run."""
import math

import numpy as np
import pytest
import torch

import oracle
from global_attention_sinks_amd import binding as Bd
from global_attention_sinks_amd import inputs as gen
from tests.gpu_util import assert_parity, dev, dev_bf16, host_f64, say
from tests.test_gpu_parity import _decode_with_positions, run_decode, run_global, run_swa
from tests.test_gpu_backward import check_grads, dsink_bar, run_fwd_bwd
from tests.test_gpu_decode_multi import run_multi
from tests.test_gpu_paged import oracle_paged, run_paged
from tests.test_gpu_varlen import check_against_oracle, run_varlen

pytestmark = pytest.mark.gpu

_rng = np.random.Generator(np.random.PCG64(20261204))


def _cfg(hq, hkv, window, base):
    return Bd.MimoAttnCfg(hq, hkv, 192, 128, 64, base, 1.0 / math.sqrt(192.0), 0.707, window)


def _swa_cases(n):
    heads = [(64, 8), (32, 8), (16, 4), (64, 16)]
    out = []
    for _ in range(n):
        out.append((int(_rng.integers(1, 4)), int(_rng.integers(1, 701)), int(_rng.integers(0, 2_000_001)),
                    int(_rng.choice([1, 7, 33, 64, 127, 128, 129, 200])), bool(_rng.integers(0, 2)),
                    heads[int(_rng.integers(0, len(heads)))]))
    return out


def _global_cases(n):
    heads = [(64, 4), (64, 8), (16, 4)]
    out = []
    for _ in range(n):
        tk = int(_rng.integers(1, 1201))
        out.append((int(_rng.integers(1, 3)), tk, int(_rng.integers(0, tk)), heads[int(_rng.integers(0, 3))],
                    bool(_rng.integers(0, 2))))
    return out


def _decode_cases(n):
    out = []
    for _ in range(n):
        window = int(_rng.choice([0, 128]))
        S = int(_rng.integers(1, 41))
        cap = 128 if window else int(_rng.integers(64, 3001))
        hkv = 8 if window else int(_rng.choice([4, 8]))
        out.append((S, cap, hkv, window, int(_rng.integers(0, 1 << 20))))
    return out


def _backward_cases(n):
    # window 1 without a sink has exactly zero dq and dk (each query sees only itself):
    # that case is tests/test_gpu_backward.py's, with a bar derived for it
    out = []
    for _ in range(n):
        B, T, w = int(_rng.integers(1, 3)), int(_rng.integers(1, 401)), int(_rng.choice([1, 16, 100, 128]))
        sinks, pos0 = bool(_rng.integers(0, 2)), int(_rng.integers(0, 100_001))
        out.append((B, T, w, sinks or w == 1, pos0))
    return out


def _varlen_cases(n):
    out = []
    for _ in range(n):
        nseq = int(_rng.integers(2, 7))
        lens_q = [int(x) for x in _rng.integers(0, 401, size=nseq)]
        lens_q[int(_rng.integers(0, nseq))] = max(lens_q) + 1     # at least one non-empty sequence
        sliding = bool(_rng.integers(0, 2))
        if sliding:
            prefix = [0] * nseq
            k_pos0 = [int(x) for x in _rng.integers(0, 300_001, size=nseq)]
        else:   # global chunks after prefixes of their own, keys from position 0
            prefix = [int(x) for x in _rng.integers(0, 600, size=nseq)]
            k_pos0 = [0] * nseq
        out.append((sliding, tuple(lens_q), tuple(prefix), tuple(k_pos0), bool(_rng.integers(0, 2))))
    return out


def _multi_cases(n):
    out = []
    for _ in range(n):
        nq, window = int(_rng.integers(2, 9)), int(_rng.choice([0, 128]))
        S = int(_rng.integers(1, 25))
        out.append((nq, window, S, int(_rng.integers(0, 1 << 20))))
    return out


def _paged_cases(n):
    out = []
    for _ in range(n):
        out.append((str(_rng.choice(["bf16", "fp8"])), int(_rng.choice([32, 64, 128, 256])), int(_rng.integers(1, 5)),
                    int(_rng.choice([0, 128])), int(_rng.integers(1, 17)), int(_rng.integers(0, 1 << 20))))
    return out


SWA = _swa_cases(8)
GLOBAL = _global_cases(6)
DECODE = _decode_cases(4)
BACKWARD = _backward_cases(4)
VARLEN = _varlen_cases(4)
MULTI = _multi_cases(4)
PAGED = _paged_cases(4)


@pytest.mark.parametrize("B,T,pos0,window,with_sinks,heads", SWA)
def test_random_prefill_swa(B, T, pos0, window, with_sinks, heads):
    hq, hkv = heads
    say(f"random prefill_swa B={B} T={T} pos0={pos0} W={window} sinks={with_sinks} heads={heads}")
    d = gen.prefill_inputs(B, T, hq, hkv, seed=7000 + T + window, with_sinks=with_sinks)
    got, lse = run_swa(d, hq, hkv, window, pos0=pos0, want_lse=True)
    ref, rlse = oracle.prefill_swa(d["q"], d["k"], d["v"], d["sinks"], pos0=pos0, window=window, base=1e4,
                                   want_lse=True)
    assert_parity(got, ref, "out")
    assert np.max(np.abs(lse - rlse.transpose(0, 2, 1))) < 1e-2


@pytest.mark.parametrize("B,Tk,q_pos0,heads,images", GLOBAL)
def test_random_prefill_global(B, Tk, q_pos0, heads, images):
    hq, hkv = heads
    say(f"random prefill_global B={B} Tk={Tk} q_pos0={q_pos0} heads={heads} images={images}")
    d = gen.prefill_inputs(B, Tk, hq, hkv, seed=7100 + Tk, with_sinks=False)
    q = d["q"][:, q_pos0:]
    got, lse = run_global(q, d["k"], d["v"], hq, hkv, q_pos0=q_pos0, want_lse=True, images=images)
    ref, rlse = oracle.prefill_global(q, d["k"], d["v"], q_pos0=q_pos0, base=1e7, want_lse=True)
    assert_parity(got, ref, "out")
    assert np.max(np.abs(lse - rlse.transpose(0, 2, 1))) < 1e-2


@pytest.mark.parametrize("S,cap,hkv,window,seed", DECODE)
def test_random_decode(S, cap, hkv, window, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = rng.integers(0, 131072 if window else cap, size=S)
    say(f"random decode S={S} cap={cap} hkv={hkv} window={window}")
    d = _decode_with_positions(S, cap, 64, hkv, 7200 + S, window, pos, window > 0)
    base = 1e4 if window else 1e7
    got = run_decode(d, 64, hkv, window, base, cap)
    ref = oracle.decode(d["q"], d["pos"], d["k_cache"], d["v_cache"], sinks=d["sinks"], window=window, base=base)
    assert_parity(got, ref, "out")


@pytest.mark.parametrize("B,T,window,with_sinks,pos0", BACKWARD)
def test_random_backward(B, T, window, with_sinks, pos0):
    say(f"random backward B={B} T={T} window={window} sinks={with_sinks} pos0={pos0}")
    d = gen.prefill_inputs(B, T, 64, 8, seed=7300 + T, with_sinks=with_sinks)
    dout = gen.normal_bf16(np.random.SeedSequence(7301 + T), (B, T, 64, 128))
    cfg = _cfg(64, 8, window, 1e4)
    got = run_fwd_bwd(d, dout, cfg, pos0=pos0)
    ref = oracle.prefill_backward(d["q"], d["k"], d["v"], dout, sinks=d["sinks"], pos0=pos0, window=window,
                                  base=1e4)
    bar = dsink_bar(d, dout, got[4], cfg, pos0) if with_sinks else None
    check_grads(got, ref, "random", bar)


@pytest.mark.parametrize("sliding,lens_q,prefix,k_pos0,images", VARLEN)
def test_random_varlen(sliding, lens_q, prefix, k_pos0, images):
    lens_k = [q + p for q, p in zip(lens_q, prefix)]
    if sliding:
        cfg, hkv, sinks = _cfg(64, 8, 128, 1e4), 8, True
    else:
        cfg, hkv, sinks = _cfg(64, 4, 0, 1e7), 4, False
    say(f"random varlen sliding={sliding} lens_q={lens_q} prefix={prefix} images={images}")
    d = gen.varlen_inputs(list(lens_q), lens_k, 64, hkv, seed=7400 + sum(lens_q), with_sinks=sinks,
                          k_pos0=list(k_pos0))
    out, lse = run_varlen(d, cfg, images=images)
    check_against_oracle(d, cfg, out, lse, "random varlen")


@pytest.mark.parametrize("nq,window,S,seed", MULTI)
def test_random_decode_multi(nq, window, S, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    if window:
        cap, hkv, base = window + nq - 1, 8, 1e4
        pos = rng.integers(0, 131072, size=S)
    else:
        cap, hkv, base = int(rng.integers(16, 3001)), 4, 1e7
        pos = rng.integers(0, cap, size=S)
    say(f"random decode_multi nq={nq} window={window} S={S} cap={cap}")
    d = gen.decode_multi_inputs(S, nq, cap, 64, hkv, seed=7500 + S, window=window, pos=pos, with_sinks=window > 0)
    got = run_multi(d, _cfg(64, hkv, window, base), cap)
    ref = oracle.decode_multi(d["q"], d["pos"], d["k_cache"], d["v_cache"], sinks=d["sinks"], window=window, base=base)
    assert_parity(got, ref, "out")


@pytest.mark.parametrize("kv,bs,nq,window,S,seed", PAGED)
def test_random_paged(kv, bs, nq, window, S, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    hkv, base = (8, 1e4) if window else (4, 1e7)
    pos = rng.integers(0, 200000 if window else 6000, size=S)
    say(f"random paged {kv} block={bs} nq={nq} window={window} S={S}")
    d = gen.paged_decode_inputs(S, nq, bs, 64, hkv, seed=7600 + S, window=window, pos=pos, with_sinks=window > 0,
                                kv_dtype=kv, k_scale=0.03, v_scale=0.04)
    cfg = _cfg(64, hkv, window, base)
    assert_parity(run_paged(d, cfg), oracle_paged(d, cfg), "out")
