"""GPU parity of the prefill backward (dq, dk, dv, d sink) against the fp64
oracle's chain-rule gradients on the same seeded inputs.  The GPU backward
takes the GPU forward's output and LSE, as a trainer would.  Bar for dq, dk,
dv: |error| <= 2e-2 + 2^-7 |ref| per element and mean-abs <= 2e-3 -- gradients
are not bounded by the values as outputs are, and a bf16 value near 8 alone
rounds by up to 1.6e-2.  d sink_h = -sum_r p_sink(r) D(r) sums every row
of the head, and the backward forms D(r) = <dO(r), O(r)> from the forward's
stored bf16 output O instead of the exact o, so its bar is that error carried
through: |error| <= sum_r p_sink(r) <|dO(r)|, |O(r) - o(r)|> + 1 % of the
reference (fp32 sums) + 1e-3."""
import math

import numpy as np
import pytest
import torch

import oracle
from global_attention_sinks_amd import binding as Bd
from global_attention_sinks_amd import inputs as gen
from tests.gpu_util import assert_grad_parity, dev, dev_bf16, host_bits, host_f64, say

pytestmark = pytest.mark.gpu


def cfg_for(hq, hkv, window, base):
    return Bd.MimoAttnCfg(hq, hkv, 192, 128, 64, base, 1.0 / math.sqrt(192.0), 0.707, window)


def dsink_bar(d, dout, out_gpu, cfg, pos0):
    """Per head: sum over rows of p_sink * <|dO|, |O_gpu - o|>, from the oracle's o and p_sink."""
    B, T = d["q"].shape[:2]
    pos = pos0 + np.arange(T, dtype=np.int64)
    bar = np.zeros(d["q"].shape[2])
    for b in range(B):
        o, ps = oracle.attention(d["q"][b], pos, d["k"][b], pos, d["v"][b], sinks=d["sinks"], window=cfg.window,
                                 base=cfg.rope_base, want_psink=True)
        dev_o = np.abs(host_f64(out_gpu[b]) - o)                         # [T, Hq, 128]
        dO = np.abs(gen.bf16_bits_to_f32(dout[b]).astype(np.float64))
        bar += np.sum(ps * np.sum(dO * dev_o, axis=2), axis=0)
    return bar


def run_fwd_bwd(d, dout, cfg, pos0=0):
    B, T, hq = d["q"].shape[:3]
    hkv = d["k"].shape[2]
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    sinks = None if d["sinks"] is None else dev(d["sinks"])
    out = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq, T), dtype=torch.float32, device="cuda")
    if cfg.window > 0:
        Bd.mimo_attn_prefill_swa(cfg, q, k, v, sinks, out, pos0=pos0, lse=lse)
    else:
        assert pos0 == 0 and sinks is None
        Bd.mimo_attn_prefill_global(cfg, q, k, v, out, lse=lse)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dsinks = torch.empty(hq, dtype=torch.float32, device="cuda") if sinks is not None else None
    Bd.mimo_attn_prefill_backward(cfg, q, k, v, sinks, out, lse, dev_bf16(dout), dq, dk, dv, dsinks, pos0=pos0)
    torch.cuda.synchronize()
    return dq, dk, dv, dsinks, out


def check_grads(got, ref, what, bar=None):
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_grad_parity(host_f64(g), r, f"{what} {name}")
    if ref[3] is not None:
        gs = got[3].cpu().numpy().astype(np.float64)
        err = np.abs(gs - ref[3])
        say(f"    dsinks: max-abs {err.max():.3e} (max |ref| {np.abs(ref[3]).max():.3e})")
        allowed = bar + 1e-2 * np.abs(ref[3]) + 1e-3
        say(f"    dsinks: worst error / allowed {np.max(err / allowed):.3f}")
        assert np.all(err <= allowed)


@pytest.mark.parametrize("B,T,window,sinks,pos0", [(2, 300, 128, True, 0), (1, 517, 128, True, 100000),
                                                   (1, 200, 16, True, 7), (1, 97, 1, True, 0),
                                                   (2, 160, 128, False, 0),
                                                   # dk/dv takes keys 16 to a wave: a window and a
                                                   # length that end inside a wave, a single token
                                                   (1, 17, 7, True, 0), (3, 48, 33, True, 0),
                                                   (1, 1, 128, True, 3),
                                                   # long enough for many stages per dk/dv workgroup
                                                   # and of dq's double-buffered key tiles
                                                   (2, 2048, 128, True, 4096)])
def test_backward_sliding(B, T, window, sinks, pos0):
    d = gen.prefill_inputs(B, T, 64, 8, seed=10001 + T, with_sinks=sinks)
    dout = gen.normal_bf16(np.random.SeedSequence(10002 + T), (B, T, 64, 128))
    say(f"backward sliding B={B} T={T} window={window} sinks={sinks} pos0={pos0}")
    got = run_fwd_bwd(d, dout, cfg_for(64, 8, window, 1e4), pos0=pos0)
    ref = oracle.prefill_backward(d["q"], d["k"], d["v"], dout, sinks=d["sinks"], pos0=pos0, window=window,
                                  base=1e4)
    bar = dsink_bar(d, dout, got[4], cfg_for(64, 8, window, 1e4), pos0) if sinks else None
    check_grads(got, ref, "sliding", bar)


@pytest.mark.parametrize("hq,hkv,T", [(64, 4, 300), (16, 4, 130), (8, 2, 70), (64, 1, 90),
                                      (16, 4, 2048)])   # 64 key tiles per dq block at the end
def test_backward_global(hq, hkv, T):
    d = gen.prefill_inputs(1, T, hq, hkv, seed=10101 + T, with_sinks=False)
    dout = gen.normal_bf16(np.random.SeedSequence(10102 + T), (1, T, hq, 128))
    say(f"backward global hq={hq} hkv={hkv} T={T}")
    got = run_fwd_bwd(d, dout, cfg_for(hq, hkv, 0, 1e7))
    ref = oracle.prefill_backward(d["q"], d["k"], d["v"], dout, window=0, base=1e7)
    check_grads(got, ref, "global")


def test_backward_window1_without_sink():
    """Window 1 and no sink: every query sees only its own key, P = 1 and dS = dP - D with
    D = dP, so the exact dq and dk are zero.  The kernels form D from the forward's stored
    bf16 output (reading r21), so their dS is that output's rounding carried through
    <dO, O>: |dS_gpu| <= sum |dO| |O_gpu - o| per (row, head), o the oracle's output.  dq
    and dk are held element by element to scale * that bound * the norm of the rotated key
    (query) pair the element mixes with its partner, with 2^-7 for the bf16 rounding of dS
    and of the result; dv = v_scale dO at the usual bar."""
    T, pos0, hq, hkv = 324, 63783, 64, 8
    d = gen.prefill_inputs(1, T, hq, hkv, seed=10301, with_sinks=False)
    dout = gen.normal_bf16(np.random.SeedSequence(10302), (1, T, hq, 128))
    cfg = cfg_for(hq, hkv, 1, 1e4)
    say(f"backward window 1, no sink: T={T} pos0={pos0}")
    got = run_fwd_bwd(d, dout, cfg, pos0=pos0)
    ref = oracle.prefill_backward(d["q"], d["k"], d["v"], dout, sinks=None, pos0=pos0, window=1, base=1e4)
    assert_grad_parity(host_f64(got[2]), ref[2], "window-1 dv")
    pos = pos0 + np.arange(T, dtype=np.int64)
    o = oracle.attention(d["q"][0], pos, d["k"][0], pos, d["v"][0], window=1, base=1e4)
    dO = np.abs(gen.bf16_bits_to_f32(dout[0]).astype(np.float64))
    ds_bound = np.sum(dO * np.abs(host_f64(got[4][0]) - o), axis=2)          # [T, Hq]
    qr = oracle.rope_partial(d["q"][0], pos, 1e4)                            # [T, Hq, 192] rotated
    kr = oracle.rope_partial(d["k"][0], pos, 1e4)                            # [T, Hkv, 192]

    def pair_norm(x):   # per element: |(x_d, x_partner)| for rotated dims, |x_d| past them
        n = np.abs(x).copy()
        r = np.sqrt(x[..., :32] ** 2 + x[..., 32:64] ** 2)
        n[..., :32] = r
        n[..., 32:64] = r
        return n

    scale, slack = cfg.softmax_scale, 1.0 + 2.0 ** -7
    G = hq // hkv
    allow_dq = slack * scale * ds_bound[:, :, None] * np.repeat(pair_norm(kr), G, axis=1) + 1e-6
    allow_dk = slack * scale * np.sum((ds_bound[:, :, None] * pair_norm(qr)).reshape(T, hkv, G, 192), axis=2) + 1e-6
    for name, g, r, allow in (("dq", got[0], ref[0], allow_dq), ("dk", got[1], ref[1], allow_dk)):
        err = np.abs(host_f64(g)[0] - r[0])
        assert np.max(np.abs(r)) < 1e-9, name                                 # exactly zero up to fp64 rounding
        say(f"  {name}: max-abs {err.max():.3e}, worst error / allowed {np.max(err / allow):.3f}")
        assert np.all(err <= allow), name


def test_backward_is_deterministic():
    d = gen.prefill_inputs(1, 256, 64, 8, seed=10201, with_sinks=True)
    dout = gen.normal_bf16(np.random.SeedSequence(10202), (1, 256, 64, 128))
    cfg = cfg_for(64, 8, 128, 1e4)
    a = run_fwd_bwd(d, dout, cfg)
    b = run_fwd_bwd(d, dout, cfg)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(host_bits(x), host_bits(y))
    assert torch.equal(a[3], b[3])
