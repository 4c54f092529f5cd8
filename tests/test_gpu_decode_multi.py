"""GPU parity of multi-query decode (several draft tokens per sequence verified
together, each attending causally to the cache) against the fp64 oracle.
Bar: max-abs <= 2e-2 and mean-abs <= 2e-3 on bf16 outputs."""
import math

import numpy as np
import pytest
import torch

import oracle
from global_attention_sinks_amd import binding as Bd
from global_attention_sinks_amd import inputs as gen
from tests.gpu_util import assert_parity, dev, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def cfg_for(hq, hkv, window, base):
    return Bd.MimoAttnCfg(hq, hkv, 192, 128, 64, base, 1.0 / math.sqrt(192.0), 0.707, window)


def run_multi(d, cfg, cap):
    S, nq, hq = d["q"].shape[:3]
    out = torch.empty((S, nq, hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(Bd.mimo_attn_decode_multi_workspace_size(cfg, S, nq, cap), dtype=torch.uint8, device="cuda")
    Bd.mimo_attn_decode_multi(cfg, dev_bf16(d["q"]), dev(d["pos"]), dev_bf16(d["k_cache"]),
                              dev_bf16(d["v_cache"]), None if d["sinks"] is None else dev(d["sinks"]), out, ws=ws)
    torch.cuda.synchronize()
    return host_f64(out)


@pytest.mark.parametrize("nq", [2, 4, 8])
def test_multi_sliding_ring(nq):
    S, W = 40, 128
    cap = W + nq - 1
    pos = np.random.Generator(np.random.PCG64(8001 + nq)).integers(0, 131072, size=S)
    pos[:7] = [0, 1, nq - 2 if nq > 1 else 0, nq - 1, 127, 128, cap]   # drafts at negative positions, short rings
    d = gen.decode_multi_inputs(S, nq, cap, 64, 8, seed=8001 + nq, window=W, pos=pos, with_sinks=True)
    say(f"multi-query decode sliding nq={nq} S={S} cap={cap}")
    got = run_multi(d, cfg_for(64, 8, W, 1e4), cap)
    ref = oracle.decode_multi(d["q"], d["pos"], d["k_cache"], d["v_cache"], sinks=d["sinks"], window=W, base=1e4)
    assert_parity(got, ref, "out")


@pytest.mark.parametrize("nq", [2, 4, 5, 8])
@pytest.mark.parametrize("with_sinks", [False, True])
def test_multi_global(nq, with_sinks):
    cap = 9000
    lens = [1, 3, 100, 2048, 2049, 5000, 9000]
    pos = np.array([L - 1 for L in lens], np.int64)
    d = gen.decode_multi_inputs(len(lens), nq, cap, 64, 4, seed=8010 + nq, window=0, pos=pos,
                                with_sinks=with_sinks)
    say(f"multi-query decode global nq={nq} lens={lens} sinks={with_sinks}")
    got = run_multi(d, cfg_for(64, 4, 0, 1e7), cap)
    ref = oracle.decode_multi(d["q"], d["pos"], d["k_cache"], d["v_cache"], sinks=d["sinks"], window=0, base=1e7)
    assert_parity(got, ref, "out")


def test_multi_equals_single_token_decodes():
    """Each draft token's row equals a one-token decode at its own position over
    the same cache (the ring keeps window + n_q - 1 slots)."""
    S, nq, W = 12, 8, 128
    cap = W + nq - 1
    pos = np.random.Generator(np.random.PCG64(8020)).integers(200, 100000, size=S)
    d = gen.decode_multi_inputs(S, nq, cap, 64, 8, seed=8020, window=W, pos=pos, with_sinks=True)
    cfg = cfg_for(64, 8, W, 1e4)
    multi = run_multi(d, cfg, cap)
    kc, vc, sk = dev_bf16(d["k_cache"]), dev_bf16(d["v_cache"]), dev(d["sinks"])
    ws = torch.empty(Bd.mimo_attn_decode_workspace_size(cfg, S, cap), dtype=torch.uint8, device="cuda")
    worst = 0.0
    for i in range(nq):
        out = torch.empty((S, 64, 128), dtype=torch.bfloat16, device="cuda")
        Bd.mimo_attn_decode(cfg, dev_bf16(np.ascontiguousarray(d["q"][:, i])), dev(pos - (nq - 1 - i)), kc, vc, sk,
                            out, ws=ws)
        torch.cuda.synchronize()
        worst = max(worst, float(np.abs(host_f64(out) - multi[:, i]).max()))
    say(f"  multi vs single-token decodes: max-abs {worst:.3e}")
    assert worst <= 1e-2
