"""GPU parity of decode over paged KV caches (block tables over shared pools)
in bf16 and fp8 e4m3, and of the paged append, against the fp64 oracle.
Bar: max-abs <= 2e-2 and mean-abs <= 2e-3 on bf16 outputs; appended bf16 rows
bit-identical to the ring append's; appended fp8 codes equal to the oracle's
except where the exact value lies within 1e-5 (relative) of a rounding
midpoint, and there one code step apart at most."""
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


def pool_dev(d, name):
    a = d[name]
    return dev(a) if a.dtype == np.uint8 else dev_bf16(a)


def run_paged(d, cfg):
    S, nq, hq = d["q"].shape[:3]
    out = torch.empty((S, nq, hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(Bd.mimo_attn_decode_multi_workspace_size(cfg, S, nq, 0), dtype=torch.uint8, device="cuda")
    Bd.mimo_attn_decode_paged(cfg, dev_bf16(d["q"]), dev(d["pos"]), pool_dev(d, "k_pool"), pool_dev(d, "v_pool"),
                              dev(d["table"]), None if d["sinks"] is None else dev(d["sinks"]), out, ws=ws,
                              k_scale=d["k_scale"], v_scale=d["v_scale"])
    torch.cuda.synchronize()
    return host_f64(out)


def oracle_paged(d, cfg, seqs=None):
    return oracle.decode_paged(d["q"], d["pos"], d["k_pool"], d["v_pool"], d["table"], block_size=d["block_size"],
                               kv_dtype=d["kv_dtype"], k_scale=d["k_scale"], v_scale=d["v_scale"], sinks=d["sinks"],
                               window=cfg.window, base=cfg.rope_base, seqs=seqs)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("nq", [1, 4])
def test_paged_global(kv, nq):
    lens = [1, 3, 100, 2048, 2049, 5000, 9000]
    pos = np.array([L - 1 for L in lens], np.int64)
    d = gen.paged_decode_inputs(len(lens), nq, 128, 64, 4, seed=9001 + nq, window=0, pos=pos, with_sinks=False,
                                kv_dtype=kv, k_scale=0.02, v_scale=0.03)
    say(f"paged global decode {kv} nq={nq} lens={lens}")
    cfg = cfg_for(64, 4, 0, 1e7)
    assert_parity(run_paged(d, cfg), oracle_paged(d, cfg), "out")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("nq,bs", [(1, 128), (8, 32), (2, 256)])
def test_paged_sliding(kv, nq, bs):
    """Sliding layers: only the blocks under some token's window are in the table
    (the others are -1), block sizes 32 to 256."""
    S = 24
    pos = np.random.Generator(np.random.PCG64(9010 + nq)).integers(0, 200000, size=S)
    pos[:5] = [0, 5, 127, 128, 300]
    d = gen.paged_decode_inputs(S, nq, bs, 64, 8, seed=9010 + nq, window=128, pos=pos, with_sinks=True,
                                kv_dtype=kv, k_scale=0.05, v_scale=0.04)
    say(f"paged sliding decode {kv} nq={nq} block={bs}")
    cfg = cfg_for(64, 8, 128, 1e4)
    assert_parity(run_paged(d, cfg), oracle_paged(d, cfg), "out")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("nq", [1, 4])
def test_paged_wide_window(kv, nq):
    """A 512-token window reads up to 18 steps: the balanced split, not one
    workgroup per sequence."""
    S, W = 20, 512
    pos = np.random.Generator(np.random.PCG64(9040 + nq)).integers(0, 100000, size=S)
    pos[:4] = [0, 300, 511, 512]
    d = gen.paged_decode_inputs(S, nq, 128, 64, 8, seed=9040 + nq, window=W, pos=pos, with_sinks=True,
                                kv_dtype=kv, k_scale=0.05, v_scale=0.04)
    say(f"paged decode window {W} {kv} nq={nq}")
    cfg = cfg_for(64, 8, W, 1e4)
    assert_parity(run_paged(d, cfg), oracle_paged(d, cfg), "out")


def test_paged_bf16_equals_per_sequence_cache_bitwise():
    """A global layer's paged bf16 cache and the same tokens in per-sequence
    caches run the same steps: identical bits."""
    lens = [700, 64, 2500]
    pos = np.array([L - 1 for L in lens], np.int64)
    d = gen.paged_decode_inputs(3, 1, 128, 64, 4, seed=9020, window=0, pos=pos, with_sinks=False)
    cap = 2560
    kc = np.full((3, cap, 4, 192), gen.BF16_NAN, np.uint16)
    vc = np.full((3, cap, 4, 128), gen.BF16_NAN, np.uint16)
    for s in range(3):
        t = np.arange(lens[s])
        kc[s, t] = d["k_pool"][d["table"][s, t // 128], t % 128]
        vc[s, t] = d["v_pool"][d["table"][s, t // 128], t % 128]
    cfg = cfg_for(64, 4, 0, 1e7)
    out = torch.empty((3, 64, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(Bd.mimo_attn_decode_workspace_size(cfg, 3, cap), dtype=torch.uint8, device="cuda")
    Bd.mimo_attn_decode(cfg, dev_bf16(np.ascontiguousarray(d["q"][:, 0])), dev(pos), dev_bf16(kc), dev_bf16(vc),
                        None, out, ws=ws)
    torch.cuda.synchronize()
    paged = run_paged(d, cfg)[:, 0]
    assert np.array_equal(host_f64(out), paged)


@pytest.mark.parametrize("block_size", [32, 128])
def test_paged_append_bf16_matches_ring_append(block_size):
    S, hkv, cap = 6, 8, 4096
    ap = gen.append_inputs(S, hkv, seed=9030, pos_lo=0, pos_hi=cap)
    pos = ap["pos"]
    cfg = cfg_for(64, hkv, 128, 1e4)
    max_blocks = cap // block_size
    table = np.arange(S * max_blocks, dtype=np.int32)[::-1].reshape(S, max_blocks).copy()   # reversed pool order
    kp = torch.zeros((S * max_blocks, block_size, hkv, 192), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((S * max_blocks, block_size, hkv, 128), dtype=torch.bfloat16, device="cuda")
    Bd.mimo_kv_paged_append(cfg, dev_bf16(ap["k"]), dev_bf16(ap["v"]), dev(pos), kp, vp, dev(table))
    kc = torch.zeros((S, cap, hkv, 192), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((S, cap, hkv, 128), dtype=torch.bfloat16, device="cuda")
    Bd.mimo_kv_ring_append(cfg, dev_bf16(ap["k"]), dev_bf16(ap["v"]), dev(pos), kc, vc)
    torch.cuda.synchronize()
    kpb, vpb, kcb, vcb = host_bits(kp), host_bits(vp), host_bits(kc), host_bits(vc)
    for s in range(S):
        p = int(pos[s])
        blk = table[s, p // block_size]
        assert np.array_equal(kpb[blk, p % block_size], kcb[s, p % cap])
        assert np.array_equal(vpb[blk, p % block_size], vcb[s, p % cap])


def test_paged_append_fp8_codes():
    S, hkv, bs, max_blocks = 16, 4, 128, 2048
    ap = gen.append_inputs(S, hkv, seed=9031, pos_lo=0, pos_hi=bs * max_blocks)
    pos = ap["pos"].copy()
    pos[:3] = [0, 1, 200000]
    ks, vs = 0.02, 0.03
    cfg = cfg_for(64, hkv, 0, 1e7)
    # each sequence's block of its new position gets its own pool block, in shuffled order
    table = np.full((S, max_blocks), -1, np.int32)
    table[np.arange(S), pos // bs] = np.random.Generator(np.random.PCG64(9031)).permutation(S)
    kp = torch.zeros((S, bs, hkv, 192), dtype=torch.uint8, device="cuda")
    vp = torch.zeros((S, bs, hkv, 128), dtype=torch.uint8, device="cuda")
    Bd.mimo_kv_paged_append(cfg, dev_bf16(ap["k"]), dev_bf16(ap["v"]), dev(pos), kp, vp, dev(table),
                            k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    kcodes, vcodes, kx, vx = oracle.kv_paged_append_fp8(ap["k"], ap["v"], pos, 1e7, ks, vs)
    kpool, vpool = kp.cpu().numpy(), vp.cpu().numpy()
    got_k = np.stack([kpool[table[s, pos[s] // bs], pos[s] % bs] for s in range(S)])
    got_v = np.stack([vpool[table[s, pos[s] // bs], pos[s] % bs] for s in range(S)])
    for name, got, want, x in (("k", got_k, kcodes, kx), ("v", got_v, vcodes, vx)):
        gv, wv = oracle.e4m3_to_f64(got), oracle.e4m3_to_f64(want)
        differ = gv != wv
        # a differing code is one step from the oracle's, at a near-midpoint value
        lo = oracle.e4m3_to_f64(oracle.e4m3_round(x * (1 - 1e-5)))
        hi = oracle.e4m3_to_f64(oracle.e4m3_round(x * (1 + 1e-5)))
        near = lo != hi
        say(f"  fp8 append {name}: {int(differ.sum())} of {differ.size} codes differ, all near a midpoint: "
            f"{bool(np.all(near[differ]))}")
        assert np.all(near[differ])
        assert np.all((gv[differ] == lo[differ]) | (gv[differ] == hi[differ]))
        assert differ.sum() <= max(3, differ.size // 10000)
