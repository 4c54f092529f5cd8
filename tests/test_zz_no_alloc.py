"""The allocation-free decode entry point (mimo_attn_decode_noalloc), called
through the C ABI, against mimo_attn_decode with a caller workspace: the same
kernels, so the outputs must agree to the parity bar (and in fact bit for bit).
Two calls in a row, the second with a smaller input, so the second runs over the
first one's leftovers in the library's scratch; then a sliding-layer ring large
enough for the split path, and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from global_attention_sinks_amd import binding as Bd
from global_attention_sinks_amd import inputs as gen
from tests.gpu_util import assert_parity, dev, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _inputs(S, cap, hkv, window, seed, pos, sinks):
    cq, ck, cv, cs, _ = gen.children(seed)
    q = gen.normal_bf16(cq, (S, 64, 192))
    kc = np.full((S, cap, hkv, 192), gen.BF16_NAN, np.uint16)
    vc = np.full((S, cap, hkv, 128), gen.BF16_NAN, np.uint16)
    ks, vs = ck.spawn(S), cv.spawn(S)
    for s in range(S):
        slots, _ = oracle.cache_slots(int(pos[s]), cap, window)
        kc[s, slots] = gen.normal_bf16(ks[s], (len(slots), hkv, 192))
        vc[s, slots] = gen.normal_bf16(vs[s], (len(slots), hkv, 128))
    return {"q": q, "pos": np.asarray(pos, np.int64), "k_cache": kc, "v_cache": vc,
            "sinks": gen.normal_f32(cs, (64,)) if sinks else None}


def _both(cfg, d):
    S = d["q"].shape[0]
    q, pos = dev_bf16(d["q"]), dev(d["pos"])
    kc, vc = dev_bf16(d["k_cache"]), dev_bf16(d["v_cache"])
    sinks = None if d["sinks"] is None else dev(d["sinks"])
    cap = d["k_cache"].shape[1]
    ws = torch.empty(Bd.mimo_attn_decode_workspace_size(cfg, S, cap), dtype=torch.uint8, device="cuda")
    ref = torch.empty((S, 64, 128), dtype=torch.bfloat16, device="cuda")
    got = torch.full((S, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    Bd.mimo_attn_decode(cfg, q, pos, kc, vc, sinks, ref, ws=ws)
    Bd.mimo_attn_decode_noalloc(cfg, q, pos, kc, vc, sinks, got)
    torch.cuda.synchronize()
    return host_f64(got), host_f64(ref)


def test_noalloc_decode_matches_workspace_decode_twice():
    cfg = Bd.global_cfg()
    rng = np.random.Generator(np.random.PCG64(7101))
    for S, cap, seed in ((16, 20000, 7102), (5, 6000, 7103)):   # second call smaller
        pos = rng.integers(1, cap, size=S) - 1
        pos[0] = cap - 1
        say(f"noalloc global decode S={S} cap={cap}")
        d = _inputs(S, cap, 4, 0, seed, pos, False)
        got, ref = _both(cfg, d)
        assert_parity(got, ref, f"noalloc vs workspace decode, S={S}")
        assert np.array_equal(got, ref)
        seqs = [0, S - 1]
        want = oracle.decode(d["q"], d["pos"], d["k_cache"], d["v_cache"], sinks=None, window=0, base=1e7,
                             seqs=seqs)
        assert_parity(got[seqs], want, f"noalloc vs oracle, S={S}")


def test_noalloc_decode_sliding_split_ring():
    """A 384-slot sliding ring (more steps than the one-workgroup-per-sequence path
    takes) goes through the split, so the scratch holds partials of 8 KV heads."""
    cfg = Bd.swa_cfg()
    S, cap = 24, 384
    pos = np.random.Generator(np.random.PCG64(7104)).integers(0, 100000, size=S)
    pos[:3] = [0, 200, 383]
    say(f"noalloc sliding decode S={S} cap={cap}")
    d = _inputs(S, cap, 8, 128, 7105, pos, True)
    got, ref = _both(cfg, d)
    assert_parity(got, ref, "noalloc vs workspace decode, sliding")
    assert np.array_equal(got, ref)


def test_noalloc_decode_rejects_more_than_its_scratch():
    lib = Bd.load_library()
    cfg = Bd.global_cfg()
    assert Bd.mimo_attn_decode_workspace_size(cfg, 752, 131072) > (32 << 20)
    assert Bd.mimo_attn_decode_workspace_size(cfg, 751, 131072) <= (32 << 20)
    fake = ctypes.c_void_p(0x10000)
    st = lib.mimo_attn_decode_noalloc(ctypes.byref(cfg), 752, fake, fake, fake, fake, 131072, None, fake, None)
    assert st == 3   # MIMO_ERR_WORKSPACE, before any launch
    assert b"scratch" in lib.mimo_last_error()


def test_noalloc_decode_in_a_captured_graph():
    """What the allocation-free call is for: captured into a HIP graph (after one
    eager call, which also looks the scratch up on this device) and replayed three
    times, with eager work and new positions between the replays; each replay
    equals the eager call on the same inputs bit for bit."""
    cfg = Bd.global_cfg()
    S, cap = 8, 5000
    rng = np.random.Generator(np.random.PCG64(7106))
    pos0 = rng.integers(1, cap, size=S) - 1
    d = _inputs(S, cap, 4, 0, 7107, np.full(S, cap - 1), False)   # every slot filled
    q, kc, vc = dev_bf16(d["q"]), dev_bf16(d["k_cache"]), dev_bf16(d["v_cache"])
    pos = dev(pos0.astype(np.int64))
    out = torch.empty((S, 64, 128), dtype=torch.bfloat16, device="cuda")
    eager = torch.empty_like(out)
    Bd.mimo_attn_decode_noalloc(cfg, q, pos, kc, vc, None, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            Bd.mimo_attn_decode_noalloc(cfg, q, pos, kc, vc, None, out)
    torch.cuda.current_stream().wait_stream(s)
    for r in range(3):
        pos.copy_(torch.from_numpy(rng.integers(0, cap, size=S).astype(np.int64)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Bd.mimo_attn_decode_noalloc(cfg, q, pos, kc, vc, None, eager)
        torch.cuda.synchronize()
        say(f"  graph replay {r}: max |replay - eager| "
            f"{(out.float() - eager.float()).abs().max().item():.3e}")
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
