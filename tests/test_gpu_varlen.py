"""GPU parity of the packed variable-length prefill (THD layout) and of chunk
continuation, against the fp64 oracle on the same seeded inputs.  Bar: max-abs
<= 2e-2 and mean-abs <= 2e-3 on bf16 outputs; LSE within 1e-2."""
import math

import numpy as np
import pytest
import torch

import oracle
from global_attention_sinks_amd import binding as Bd
from global_attention_sinks_amd import inputs as gen
from tests.gpu_util import assert_parity, dev, dev_bf16, host_bits, host_f64, say

pytestmark = pytest.mark.gpu


def cfg_for(hq, hkv, window, base):
    return Bd.MimoAttnCfg(hq, hkv, 192, 128, 64, base, 1.0 / math.sqrt(192.0), 0.707, window)


def run_varlen(d, cfg, max_q=None, want_lse=True, out_fill=None, images=True):
    """images: global layers get a tile-image workspace filled with 0xFF bytes (NaN
    bf16), so any image byte read without being written shows up."""
    total_q, hq = d["q"].shape[:2]
    ws = False
    if images:
        n = Bd.mimo_attn_prefill_workspace_size(cfg, len(d["cu_q"]) - 1, d["k"].shape[0])
        ws = torch.full((n,), 255, dtype=torch.uint8, device="cuda") if n else False
    lens_q = np.diff(d["cu_q"])
    max_q = int(lens_q.max()) if max_q is None else max_q
    out = torch.empty((total_q, hq, 128), dtype=torch.bfloat16, device="cuda")
    if out_fill is not None:
        out.fill_(out_fill)
    lse = torch.empty((hq, total_q), dtype=torch.float32, device="cuda") if want_lse else None
    Bd.mimo_attn_prefill_varlen(cfg, dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]),
                                None if d["sinks"] is None else dev(d["sinks"]), dev(d["cu_q"]),
                                dev(d["cu_k"]), max_q, out,
                                k_pos0=None if d["k_pos0"] is None else dev(d["k_pos0"]), lse=lse, ws=ws)
    torch.cuda.synchronize()
    return out, lse


def check_against_oracle(d, cfg, out, lse, what):
    ref, rlse = oracle.prefill_varlen(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], k_pos0=d["k_pos0"],
                                      sinks=d["sinks"], window=cfg.window, base=cfg.rope_base, want_lse=True)
    rows = np.concatenate([np.arange(d["cu_q"][b], d["cu_q"][b + 1]) for b in range(len(d["cu_q"]) - 1)])
    assert_parity(host_f64(out)[rows], ref[rows], what)
    if lse is not None:
        err = np.abs(lse.cpu().numpy().astype(np.float64)[:, rows] - rlse[:, rows])
        say(f"  lse max-abs {err.max():.3e}")
        assert err.max() < 1e-2


@pytest.mark.parametrize("layer", ["sliding", "global", "global-staged"])
def test_thd_ragged_sequences(layer):
    """Several packed sequences of ragged lengths (one token, tile edges, an empty
    one, several tiles), each starting at its own position."""
    lens = [1, 31, 32, 33, 0, 200, 517]
    pos0 = [0, 5, 1000, 131000, 7, 127, 262144]
    if layer == "sliding":
        cfg, hkv, sinks = cfg_for(64, 8, 128, 1e4), 8, True
    else:
        cfg, hkv, sinks = cfg_for(64, 4, 0, 1e7), 4, False
        pos0 = [0] * len(lens)   # a global chunk holding its whole prefix starts at 0
    d = gen.varlen_inputs(lens, lens, 64, hkv, seed=7001, with_sinks=sinks, k_pos0=pos0)
    say(f"varlen {layer}: lens {lens}")
    out, lse = run_varlen(d, cfg, images=layer != "global-staged")
    check_against_oracle(d, cfg, out, lse, f"{layer} THD")


def test_sliding_chunk_continuation():
    """Chunks that continue sequences: the keys are the chunk plus the 127 tokens
    before it (fewer at the start of a sequence)."""
    chunk = 300
    starts = [0, 64, 127, 128, 5000, 200000]   # position of each chunk's first query
    lens_k = [chunk + min(127, s) for s in starts]
    kpos = [s - min(127, s) for s in starts]
    d = gen.varlen_inputs([chunk] * len(starts), lens_k, 64, 8, seed=7002, with_sinks=True, k_pos0=kpos)
    say(f"sliding chunk continuation at {starts}")
    out, lse = run_varlen(d, cfg_for(64, 8, 128, 1e4))
    check_against_oracle(d, cfg_for(64, 8, 128, 1e4), out, lse, "sliding chunks")


def test_global_chunk_continuation():
    """Global chunks against their whole prefix, packed: prefixes of 0, 700 and
    1200 tokens, chunks of 300, 64 and 257 queries."""
    lens_q, prefix = [300, 64, 257], [0, 700, 1200]
    lens_k = [q + p for q, p in zip(lens_q, prefix)]
    d = gen.varlen_inputs(lens_q, lens_k, 64, 4, seed=7003, with_sinks=False)
    say(f"global chunk continuation: queries {lens_q} after prefixes {prefix}")
    out, lse = run_varlen(d, cfg_for(64, 4, 0, 1e7))
    check_against_oracle(d, cfg_for(64, 4, 0, 1e7), out, lse, "global chunks")


@pytest.mark.parametrize("layer", ["sliding", "global", "global-staged"])
def test_packed_equals_dense_bitwise(layer):
    """Dense batches and the same batches packed run the same kernel: identical bits
    (global layers with tile images, whose tiles then sit at other places of the
    workspace, and without)."""
    B, T = 2, 384
    sliding = layer == "sliding"
    ws = False if layer == "global-staged" else None
    hkv = 8 if sliding else 4
    cfg = cfg_for(64, hkv, 128 if sliding else 0, 1e4 if sliding else 1e7)
    d = gen.prefill_inputs(B, T, 64, hkv, seed=7004, with_sinks=sliding)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    dense = torch.empty((B, T, 64, 128), dtype=torch.bfloat16, device="cuda")
    dlse = torch.empty((B, 64, T), dtype=torch.float32, device="cuda")
    if sliding:
        Bd.mimo_attn_prefill_swa(cfg, q, k, v, dev(d["sinks"]), dense, lse=dlse)
    else:
        Bd.mimo_attn_prefill_global(cfg, q, k, v, dense, lse=dlse, ws=ws)
    cu = dev(np.array([0, T, 2 * T], np.int32))
    packed = torch.empty((B * T, 64, 128), dtype=torch.bfloat16, device="cuda")
    plse = torch.empty((64, B * T), dtype=torch.float32, device="cuda")
    Bd.mimo_attn_prefill_varlen(cfg, q.view(B * T, 64, 192), k.view(B * T, hkv, 192), v.view(B * T, hkv, 128),
                                dev(d["sinks"]) if sliding else None, cu, cu, T, packed, lse=plse, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dense).reshape(B * T, 64, 128), host_bits(packed))
    assert torch.equal(dlse.permute(1, 0, 2).reshape(64, B * T), plse)


def test_rows_past_max_seqlen_are_left_alone():
    """A sequence longer than max_seqlen_q gets its first max_seqlen_q rows only;
    the rest of the output is not written (and nothing is read out of bounds)."""
    lens = [100, 40]
    d = gen.varlen_inputs(lens, lens, 64, 8, seed=7005, with_sinks=True)
    out, _ = run_varlen(d, cfg_for(64, 8, 128, 1e4), max_q=64, want_lse=False, out_fill=7.0)
    got = host_f64(out)
    assert np.all(got[64:100] == 7.0)
    ref = oracle.prefill_varlen(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], sinks=d["sinks"], window=128,
                                base=1e4)
    rows = np.r_[0:64, 100:140]
    assert_parity(got[rows], ref[rows], "rows below max_seqlen_q")


def test_one_workspace_across_global_calls():
    """A tile-image workspace sized for the largest call serves calls of other shapes
    in turn (dense, packed, dense again): each call rewrites the images it reads."""
    cfg = cfg_for(64, 4, 0, 1e7)
    d1 = gen.prefill_inputs(1, 700, 64, 4, seed=7010, with_sinks=False)
    d2 = gen.varlen_inputs([40, 300, 1], [40 + 250, 300, 1], 64, 4, seed=7011, with_sinks=False)
    d3 = gen.prefill_inputs(2, 130, 64, 4, seed=7012, with_sinks=False)
    n = max(Bd.mimo_attn_prefill_workspace_size(cfg, 1, 700),
            Bd.mimo_attn_prefill_workspace_size(cfg, 3, d2["k"].shape[0]),
            Bd.mimo_attn_prefill_workspace_size(cfg, 2, 260))
    ws = torch.full((n,), 255, dtype=torch.uint8, device="cuda")

    def dense(d, q_pos0):
        B, Tk = d["k"].shape[:2]
        out = torch.empty((B, Tk - q_pos0, 64, 128), dtype=torch.bfloat16, device="cuda")
        Bd.mimo_attn_prefill_global(cfg, dev_bf16(d["q"][:, q_pos0:]), dev_bf16(d["k"]), dev_bf16(d["v"]), out,
                                    q_pos0=q_pos0, ws=ws)
        torch.cuda.synchronize()
        ref = oracle.prefill_global(d["q"][:, q_pos0:], d["k"], d["v"], q_pos0=q_pos0, base=1e7)
        return host_f64(out), ref

    say("one workspace: dense B=1 Tk=700 (chunk at 300)")
    got, ref = dense(d1, 300)
    assert_parity(got, ref, "dense 700")
    say("one workspace: packed 3 sequences")
    total_q = d2["q"].shape[0]
    out = torch.empty((total_q, 64, 128), dtype=torch.bfloat16, device="cuda")
    Bd.mimo_attn_prefill_varlen(cfg, dev_bf16(d2["q"]), dev_bf16(d2["k"]), dev_bf16(d2["v"]), None, dev(d2["cu_q"]),
                                dev(d2["cu_k"]), 300, out, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(d2["q"], d2["k"], d2["v"], d2["cu_q"], d2["cu_k"], window=0, base=1e7)
    assert_parity(host_f64(out), ref, "packed")
    say("one workspace: dense B=2 Tk=130")
    got, ref = dense(d3, 0)
    assert_parity(got, ref, "dense 2 x 130")
