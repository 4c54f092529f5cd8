"""Parity at the workloads' full sizes, in the launch configuration bench.py
times, checked against the fp64 oracle on sampled output rows (the oracle
computes rows one by one); every output is also checked to be finite.

  * sliding-window + sink prefill, B=4 x T=8192
  * global causal prefill, T=32768
  * mixed decode step: 64 sliding sequences (ring of 128) + 16 global
    sequences (KV lengths ~U[32768, 131072], cap 131072), NaN in unused slots
  * long global prefill T=524288 in query chunks of 65536: all 8 chunks, each
    against its whole prefix, 32 stratified rows of each
  * multi-query decode: 64 sliding sequences x 8 draft tokens, 16 global x 4
  * paged fp8 decode (128-slot blocks in shuffled pools): the 16 global
    sequences of the mixed decode and 64 sliding sequences
  * sliding-window + sink backward, B=4 x T=8192: dq, dk, dv of every token and
    d sink over all rows
  * serving chunks of 8192 tokens, packed: four sliding-window chunks that
    continue sequences (127 earlier keys each) and four global chunks against
    prefixes of up to 57344 tokens
"""
import numpy as np
import pytest
import torch

import oracle
from global_attention_sinks_amd import binding as Bd
from global_attention_sinks_amd import inputs as gen
from tests.gpu_util import assert_grad_parity, assert_parity, dev, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def sample_rows(T, extra, seed, must=()):
    rng = np.random.default_rng(seed)
    base = [0, 1, 31, 32, 63, 64, 127, 128, T // 2, T - 2, T - 1, *must]
    return np.unique(np.clip(np.concatenate([base, rng.integers(0, T, extra)]), 0, T - 1))


def test_swa_prefill_b4_t8192():
    say("full-size sliding prefill B=4 T=8192")
    d = gen.prefill_inputs(4, 8192, 64, 8, seed=1001, with_sinks=True)
    out = torch.empty((4, 8192, 64, 128), dtype=torch.bfloat16, device="cuda")
    Bd.mimo_attn_prefill_swa(Bd.swa_cfg(), dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]),
                             dev(d["sinks"]), out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rows = sample_rows(8192, 40, 1)
    got = host_f64(out[:, torch.from_numpy(rows).cuda()])
    ref = oracle.prefill_swa(d["q"], d["k"], d["v"], d["sinks"], window=128, base=1e4, rows=rows)
    assert_parity(got, ref, f"{len(rows)} rows x 4 seqs")


@pytest.mark.parametrize("images", [True, False], ids=["images", "staged"])
def test_global_prefill_t32768(images):
    say(f"full-size global prefill T=32768 images={images}")
    d = gen.prefill_inputs(1, 32768, 64, 4, seed=1002, with_sinks=False)
    out = torch.empty((1, 32768, 64, 128), dtype=torch.bfloat16, device="cuda")
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    Bd.mimo_attn_prefill_global(Bd.global_cfg(), q, k, v, out, ws=None if images else False)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    if images:   # the key-norm bound that decides the skipped row maxima is summed in a fixed order
        again = torch.empty_like(out)
        Bd.mimo_attn_prefill_global(Bd.global_cfg(), q, k, v, again)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "not bitwise repeatable"
    rows = sample_rows(32768, 12, 2, must=(16383, 16384))
    got = host_f64(out[:, torch.from_numpy(rows).cuda()])
    ref = oracle.prefill_global(d["q"], d["k"], d["v"], base=1e7, rows=rows)
    assert_parity(got, ref, f"{len(rows)} rows")


def test_mixed_decode_full():
    say("full-size mixed decode: 64 sliding + 16 global sequences")
    for name, S, cap, hkv, window, base, lo, hi, sinks, seed, check in (
            ("sliding", 64, 128, 8, 128, 1e4, 128, 131072, True, 1003, list(range(64))),
            ("global", 16, 131072, 4, 0, 1e7, 32768, 131072, False, 2003, list(range(16)))):
        dd = gen.decode_inputs(S, cap, 64, hkv, seed=seed, window=window, pos_lo=lo, pos_hi=hi,
                               with_sinks=sinks)
        cfg = Bd.swa_cfg() if window else Bd.global_cfg()
        ws = torch.empty(max(1, Bd.mimo_attn_decode_workspace_size(cfg, S, cap)), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty((S, 64, 128), dtype=torch.bfloat16, device="cuda")
        Bd.mimo_attn_decode(cfg, dev_bf16(dd["q"]), dev(dd["pos"]), dev_bf16(dd["k_cache"]),
                            dev_bf16(dd["v_cache"]), dev(dd["sinks"]) if sinks else None, out, ws=ws)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
        got = host_f64(out)[check]
        ref = oracle.decode(dd["q"], dd["pos"], dd["k_cache"], dd["v_cache"], sinks=dd["sinks"],
                            window=window, base=base, seqs=check)
        assert_parity(got, ref, f"{name} decode, {len(check)} of {S} sequences")


LONG_T, LONG_C = 524288, 65536


@pytest.fixture(scope="module")
def long_prefill_kv():
    """Keys and values 0..524287 of the long prefill, drawn as
    prefill_inputs(1, 524288, ...) draws them, on the host and the device."""
    say("drawing k/v of the 524288-token prefill")
    kv = gen.global_prefill_chunk(LONG_T, 64, 4, seed=1004, t_lo=LONG_T, t_hi=LONG_T)   # no query rows
    full = {"k": kv["k"], "v": kv["v"]}
    full["k_dev"], full["v_dev"] = dev_bf16(full["k"]), dev_bf16(full["v"])
    ws = Bd.mimo_attn_prefill_workspace_size(Bd.global_cfg(), 1, LONG_T)
    full["ws"] = torch.empty(ws, dtype=torch.uint8, device="cuda")
    yield full
    del full


def stratified_rows(C, n, seed):
    """n query rows of a chunk: its first and last rows, both sides of its
    middle and of 32- and 64-row block edges near its ends, and one row from
    each of the remaining equal strata."""
    fixed = [0, 1, 31, 32, 63, 64, C // 2 - 1, C // 2, C - 65, C - 64, C - 2, C - 1]
    rng = np.random.default_rng(seed)
    k = n - len(fixed)
    edges = np.linspace(0, C, k + 1).astype(np.int64)
    strata = [int(rng.integers(edges[i], edges[i + 1])) for i in range(k)]
    rows = np.unique(np.array(fixed + strata, dtype=np.int64))
    assert len(rows) == n
    return rows


@pytest.mark.parametrize("chunk", range(8))
def test_long_global_prefill_chunk(chunk, long_prefill_kv):
    """Chunk c of the 524288-token prefill (queries 65536c .. 65536(c+1)-1 against
    keys 0 .. 65536(c+1)-1) in the launch configuration the benchmark times (one
    tile-image workspace for the whole prefix); 32 stratified rows x 64 heads."""
    lo, hi = chunk * LONG_C, (chunk + 1) * LONG_C
    say(f"full-size long prefill T={LONG_T}: chunk {chunk} (queries {lo}..{hi - 1}, keys 0..{hi - 1})")
    q = gen.global_prefill_chunk(LONG_T, 64, 4, seed=1004, t_lo=lo, t_hi=hi, kv=False)["q"]
    kv = long_prefill_kv
    out = torch.empty((1, LONG_C, 64, 128), dtype=torch.bfloat16, device="cuda")
    Bd.mimo_attn_prefill_global(Bd.global_cfg(), dev_bf16(q), kv["k_dev"][:, :hi], kv["v_dev"][:, :hi], out,
                                q_pos0=lo, ws=kv["ws"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rows = stratified_rows(LONG_C, 32, 100 + chunk)
    got = host_f64(out[:, torch.from_numpy(rows).cuda()])
    ref = oracle.prefill_global(q, kv["k"][:, :hi], kv["v"][:, :hi], q_pos0=lo, base=1e7, rows=rows)
    assert_parity(got, ref, f"chunk {chunk}, {len(rows)} rows x 64 heads")


def test_packed_serving_chunks():
    chunk = 8192
    for layer, seed in (("sliding", 1005), ("global", 1006)):
        if layer == "sliding":
            starts = [8192, 65536, 131072, 262144]
            lens_k = [chunk + 127] * 4
            kpos = [st - 127 for st in starts]
            d = gen.varlen_inputs([chunk] * 4, lens_k, 64, 8, seed=seed, with_sinks=True, k_pos0=kpos)
            cfg = Bd.swa_cfg()
        else:
            prefix = [0, 8192, 24576, 57344]
            d = gen.varlen_inputs([chunk] * 4, [chunk + p for p in prefix], 64, 4, seed=seed, with_sinks=False)
            cfg = Bd.global_cfg()
        say(f"full-size packed serving chunks: {layer}")
        out = torch.empty((4 * chunk, 64, 128), dtype=torch.bfloat16, device="cuda")
        Bd.mimo_attn_prefill_varlen(cfg, dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]),
                                    None if d["sinks"] is None else dev(d["sinks"]), dev(d["cu_q"]),
                                    dev(d["cu_k"]), chunk, out,
                                    k_pos0=None if d["k_pos0"] is None else dev(d["k_pos0"]))
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
        got_all = host_f64(out)
        for b in range(4):
            rows = sample_rows(chunk, 6, 10 + b)
            q0, k0 = int(d["cu_q"][b]), int(d["cu_k"][b])
            lq, lk = chunk, int(d["cu_k"][b + 1]) - k0
            p0 = 0 if d["k_pos0"] is None else int(d["k_pos0"][b])
            kp = p0 + np.arange(lk, dtype=np.int64)
            ref = oracle.attention(d["q"][q0 + rows], kp[lk - lq + rows], d["k"][k0:k0 + lk], kp,
                                   d["v"][k0:k0 + lk], sinks=d["sinks"], window=cfg.window, base=cfg.rope_base)
            assert_parity(got_all[q0 + rows], ref, f"{layer} chunk {b}, {len(rows)} rows")


def test_multi_query_decode_full():
    """Speculative verification at the mixed-decode sizes: 64 sliding sequences
    with 8 draft tokens (ring of 135) and 16 global sequences with 4."""
    for name, S, nq, cap, hkv, window, base, sinks, seed, check in (
            ("sliding", 64, 8, 135, 8, 128, 1e4, True, 1007, list(range(0, 64, 4))),
            ("global", 16, 4, 131072, 4, 0, 1e7, False, 1008, [0, 7, 15])):
        rng = np.random.Generator(np.random.PCG64(seed))
        if window:
            pos = rng.integers(128, 131072, size=S)
        else:
            pos = rng.integers(32768, 131072, size=S, endpoint=True) - 1
        say(f"full-size multi-query decode: {name}, {S} sequences x {nq} tokens")
        dd = gen.decode_multi_inputs(S, nq, cap, 64, hkv, seed=seed, window=window, pos=pos, with_sinks=sinks)
        cfg = Bd.swa_cfg() if window else Bd.global_cfg()
        ws = torch.empty(Bd.mimo_attn_decode_multi_workspace_size(cfg, S, nq, cap), dtype=torch.uint8, device="cuda")
        out = torch.empty((S, nq, 64, 128), dtype=torch.bfloat16, device="cuda")
        Bd.mimo_attn_decode_multi(cfg, dev_bf16(dd["q"]), dev(dd["pos"]), dev_bf16(dd["k_cache"]),
                                  dev_bf16(dd["v_cache"]), dev(dd["sinks"]) if sinks else None, out, ws=ws)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
        got = host_f64(out)[check]
        ref = oracle.decode_multi(dd["q"], dd["pos"], dd["k_cache"], dd["v_cache"], sinks=dd["sinks"],
                                  window=window, base=base, seqs=check)
        assert_parity(got, ref, f"{name}, {len(check)} of {S} sequences")


def test_paged_fp8_decode_full():
    for name, S, hkv, window, base, sinks, seed, check in (
            ("global", 16, 4, 0, 1e7, False, 1009, [0, 6, 11, 15]),
            ("sliding", 64, 8, 128, 1e4, True, 1010, list(range(0, 64, 8)))):
        rng = np.random.Generator(np.random.PCG64(seed))
        if window:
            pos = rng.integers(128, 131072, size=S)
        else:
            pos = rng.integers(32768, 131072, size=S, endpoint=True) - 1
        say(f"full-size paged fp8 decode: {name}, {S} sequences")
        d = gen.paged_decode_inputs(S, 1, 128, 64, hkv, seed=seed, window=window, pos=pos, with_sinks=sinks,
                                    kv_dtype="fp8", k_scale=0.02, v_scale=0.03)
        cfg = Bd.swa_cfg() if window else Bd.global_cfg()
        out = torch.empty((S, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(Bd.mimo_attn_decode_multi_workspace_size(cfg, S, 1, 0), dtype=torch.uint8, device="cuda")
        Bd.mimo_attn_decode_paged(cfg, dev_bf16(d["q"]), dev(d["pos"]), dev(d["k_pool"]), dev(d["v_pool"]),
                                  dev(d["table"]), dev(d["sinks"]) if sinks else None, out, ws=ws,
                                  k_scale=0.02, v_scale=0.03)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
        got = host_f64(out)[check]
        ref = oracle.decode_paged(d["q"], d["pos"], d["k_pool"], d["v_pool"], d["table"], block_size=128,
                                  kv_dtype="fp8", k_scale=0.02, v_scale=0.03, sinks=d["sinks"], window=window,
                                  base=base, seqs=check)
        assert_parity(got, ref, f"{name}, {len(check)} of {S} sequences")


def test_swa_backward_b4_t8192():
    """The B4 x T8192 sliding-window + sink backward compared in full: dq, dk, dv of
    every token of every sequence, and d sink summed over all 32768 rows of each
    head (its bar carries the forward's stored-output error, as in
    tests/test_gpu_backward.py)."""
    from tests.test_gpu_backward import dsink_bar
    say("full-size sliding backward B=4 T=8192")
    B, T = 4, 8192
    d = gen.prefill_inputs(B, T, 64, 8, seed=1011, with_sinks=True)
    dout = gen.normal_bf16(np.random.SeedSequence(1012), (B, T, 64, 128))
    cfg = Bd.swa_cfg()
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    sinks = dev(d["sinks"])
    out = torch.empty((B, T, 64, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 64, T), dtype=torch.float32, device="cuda")
    Bd.mimo_attn_prefill_swa(cfg, q, k, v, sinks, out, lse=lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsinks = torch.empty(64, dtype=torch.float32, device="cuda")
    Bd.mimo_attn_prefill_backward(cfg, q, k, v, sinks, out, lse, dev_bf16(dout), dq, dk, dv, dsinks)
    torch.cuda.synchronize()
    for t_ in (dq, dk, dv, dsinks):
        assert bool(torch.isfinite(t_).all())
    pos = np.arange(T, dtype=np.int64)
    ds_ref = np.zeros(64)
    for b in range(B):
        say(f"  oracle backward of sequence {b}")
        rdq, rdk, rdv, rds = oracle.attention_backward(d["q"][b], pos, d["k"][b], pos, d["v"][b], dout[b],
                                                       sinks=d["sinks"], window=128, base=1e4)
        ds_ref += rds
        for name, got, ref in (("dq", host_f64(dq[b]), rdq), ("dk", host_f64(dk[b]), rdk),
                               ("dv", host_f64(dv[b]), rdv)):
            assert_grad_parity(got, ref, f"seq {b} {name}")
    bar = dsink_bar(d, dout, out, cfg, 0)
    gs = dsinks.cpu().numpy().astype(np.float64)
    err = np.abs(gs - ds_ref)
    allowed = bar + 1e-2 * np.abs(ds_ref) + 1e-3
    say(f"  dsinks over 32768 rows: max-abs {err.max():.3e} (max |ref| {np.abs(ds_ref).max():.3e}); "
        f"worst error / allowed {np.max(err / allowed):.3f}")
    assert np.all(err <= allowed)
