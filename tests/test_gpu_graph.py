"""Every call of the library only enqueues kernels on the caller's stream (no allocation,
copy, memset or host synchronisation), so a whole step can be captured into one HIP graph.

The step below makes every computing call once: partial RoPE, sliding prefill with LSE and
its backward, global prefill with tile images, packed (THD) global prefill, ring append
then sliding decode, multi-query sliding decode, global split-K decode, fp8 paged append
then paged decode.  It is captured once (after an eager run, which also loads the code
objects) and replayed three times with new inputs written between replays.  After each
replay the same calls run eagerly on the same inputs into a second set of outputs and
caches; all kernels are deterministic, so every output and every cache the step writes
must equal its eager counterpart bit for bit.  Positions change between replays wherever
the buffer shapes do not depend on them (ring, global and multi-query decode)."""
import numpy as np
import pytest
import torch

from global_attention_sinks_amd import binding as Bd
from global_attention_sinks_amd import inputs as gen
from tests.gpu_util import dev, dev_bf16, say

pytestmark = pytest.mark.gpu

T_SWA, T_GLOB = 300, 200
S_RING, CAP_RING = 8, 128
S_MULTI, NQ, CAP_MULTI = 4, 4, 160
S_GDEC, CAP_GDEC = 4, 2000
S_PAGED, BS = 4, 32
PAGED_POS = np.array([0, 31, 1000, 2999], dtype=np.int64)   # fixed: the pool's shape follows them
LENS_Q, LENS_K, KPOS0 = [1, 40, 0, 97], [1, 100, 3, 97], [0, 5000, 12, 64]
K_SCALE, V_SCALE = 0.5, 0.25


def draw(r):
    """Host inputs of round r: same shapes every round, new values."""
    base = 9100 + 32 * r
    swa = gen.prefill_inputs(1, T_SWA, 64, 8, seed=base, with_sinks=True)
    glob = gen.prefill_inputs(1, T_GLOB, 64, 4, seed=base + 1, with_sinks=False)
    ring = gen.decode_inputs(S_RING, CAP_RING, 64, 8, base + 2, 128, 128, 131072, True)
    mpos = np.random.Generator(np.random.PCG64(base + 3)).integers(0, 50000, size=S_MULTI)
    multi = gen.decode_multi_inputs(S_MULTI, NQ, CAP_MULTI, 64, 8, base + 4, 128, mpos, True)
    gdec = gen.decode_inputs(S_GDEC, CAP_GDEC, 64, 4, base + 5, 0, 1000, CAP_GDEC, False)
    paged = gen.paged_decode_inputs(S_PAGED, 1, BS, 64, 4, base + 6, 0, PAGED_POS, False, "fp8", K_SCALE, V_SCALE)
    return {
        "q": swa["q"], "k": swa["k"], "v": swa["v"], "sinks": swa["sinks"],
        "dO": gen.normal_bf16(np.random.SeedSequence(base + 7), (1, T_SWA, 64, 128)),
        "tpos": np.arange(T_SWA, dtype=np.int64) + 70000 * r,
        "gq": glob["q"], "gk": glob["k"], "gv": glob["v"],
        "vl": gen.varlen_inputs(LENS_Q, LENS_K, 64, 4, base + 8, False, k_pos0=KPOS0),
        "rq": ring["q"], "rpos": ring["pos"], "rk0": ring["k_cache"], "rv0": ring["v_cache"],
        "ak": gen.append_inputs(S_RING, 8, base + 9, 0, 1),
        "mq": multi["q"], "mpos": multi["pos"], "mk": multi["k_cache"], "mv": multi["v_cache"],
        "dq_": gdec["q"], "dpos": gdec["pos"], "dk_": gdec["k_cache"], "dv_": gdec["v_cache"],
        "pq": paged["q"], "table": paged["table"], "kp0": paged["k_pool"], "vp0": paged["v_pool"],
        "pk": gen.append_inputs(S_PAGED, 4, base + 10, 0, 1),
    }


def device_inputs(h):
    vl = h["vl"]
    return {
        "q": dev_bf16(h["q"]), "k": dev_bf16(h["k"]), "v": dev_bf16(h["v"]), "sinks": dev(h["sinks"]),
        "dO": dev_bf16(h["dO"]), "tpos": dev(h["tpos"]),
        "gq": dev_bf16(h["gq"]), "gk": dev_bf16(h["gk"]), "gv": dev_bf16(h["gv"]),
        "lq": dev_bf16(vl["q"]), "lk": dev_bf16(vl["k"]), "lv": dev_bf16(vl["v"]),
        "cu_q": dev(vl["cu_q"]), "cu_k": dev(vl["cu_k"]), "kpos0": dev(vl["k_pos0"]),
        "rq": dev_bf16(h["rq"]), "rpos": dev(h["rpos"]), "rk0": dev_bf16(h["rk0"]), "rv0": dev_bf16(h["rv0"]),
        "ak": dev_bf16(h["ak"]["k"]), "av": dev_bf16(h["ak"]["v"]),
        "mq": dev_bf16(h["mq"]), "mpos": dev(h["mpos"]), "mk": dev_bf16(h["mk"]), "mv": dev_bf16(h["mv"]),
        "dq_": dev_bf16(h["dq_"]), "dpos": dev(h["dpos"]), "dk_": dev_bf16(h["dk_"]), "dv_": dev_bf16(h["dv_"]),
        "pq": dev_bf16(h["pq"]), "ppos": dev(PAGED_POS), "table": dev(h["table"]),
        "kp0": dev(h["kp0"]), "vp0": dev(h["vp0"]),
        "pk": dev_bf16(h["pk"]["k"]), "pv": dev_bf16(h["pk"]["v"]),
    }


def outputs(I):
    """One set of outputs, caches the step writes, and workspaces."""
    swa, glob = Bd.swa_cfg(), Bd.global_cfg()
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    f = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    u8 = lambda n: torch.empty(max(1, n), dtype=torch.uint8, device="cuda")
    total_q, total_k = I["lq"].shape[0], I["lk"].shape[0]
    return {
        "rope": e(T_SWA, 64, 192), "out": e(1, T_SWA, 64, 128), "lse": f(1, 64, T_SWA),
        "dq": e(1, T_SWA, 64, 192), "dk": e(1, T_SWA, 8, 192), "dv": e(1, T_SWA, 8, 128), "dsinks": f(64),
        "bws": u8(Bd.mimo_attn_backward_workspace_size(swa, 1, T_SWA)),
        "gout": e(1, T_GLOB, 64, 128), "glse": f(1, 64, T_GLOB),
        "gws": u8(Bd.mimo_attn_prefill_workspace_size(glob, 1, T_GLOB)),
        "lout": e(total_q, 64, 128), "llse": f(64, total_q),
        "lws": u8(Bd.mimo_attn_prefill_workspace_size(glob, len(LENS_Q), total_k)),
        "rk": torch.empty_like(I["rk0"]), "rv": torch.empty_like(I["rv0"]), "rout": e(S_RING, 64, 128),
        "rws": u8(Bd.mimo_attn_decode_workspace_size(swa, S_RING, CAP_RING)),
        "mout": e(S_MULTI, NQ, 64, 128), "mws": u8(Bd.mimo_attn_decode_multi_workspace_size(swa, S_MULTI, NQ, 0)),
        "dout": e(S_GDEC, 64, 128), "dws": u8(Bd.mimo_attn_decode_workspace_size(glob, S_GDEC, CAP_GDEC)),
        "kp": torch.empty_like(I["kp0"]), "vp": torch.empty_like(I["vp0"]), "pout": e(S_PAGED, 1, 64, 128),
        "pws": u8(Bd.mimo_attn_decode_multi_workspace_size(glob, S_PAGED, 1, 0)),
    }


def step(I, O):
    swa, glob = Bd.swa_cfg(), Bd.global_cfg()
    Bd.mimo_rope_partial(swa, I["q"].view(T_SWA, 64, 192), O["rope"], I["tpos"])
    Bd.mimo_attn_prefill_swa(swa, I["q"], I["k"], I["v"], I["sinks"], O["out"], lse=O["lse"])
    Bd.mimo_attn_prefill_backward(swa, I["q"], I["k"], I["v"], I["sinks"], O["out"], O["lse"], I["dO"],
                                  O["dq"], O["dk"], O["dv"], O["dsinks"], ws=O["bws"])
    Bd.mimo_attn_prefill_global(glob, I["gq"], I["gk"], I["gv"], O["gout"], lse=O["glse"], ws=O["gws"])
    Bd.mimo_attn_prefill_varlen(glob, I["lq"], I["lk"], I["lv"], None, I["cu_q"], I["cu_k"], max(LENS_Q),
                                O["lout"], k_pos0=I["kpos0"], lse=O["llse"], ws=O["lws"])
    Bd.mimo_kv_ring_append(swa, I["ak"], I["av"], I["rpos"], O["rk"], O["rv"])
    Bd.mimo_attn_decode(swa, I["rq"], I["rpos"], O["rk"], O["rv"], I["sinks"], O["rout"], ws=O["rws"])
    Bd.mimo_attn_decode_multi(swa, I["mq"], I["mpos"], I["mk"], I["mv"], I["sinks"], O["mout"], ws=O["mws"])
    Bd.mimo_attn_decode(glob, I["dq_"], I["dpos"], I["dk_"], I["dv_"], None, O["dout"], ws=O["dws"])
    Bd.mimo_kv_paged_append(glob, I["pk"], I["pv"], I["ppos"], O["kp"], O["vp"], I["table"],
                            k_scale=K_SCALE, v_scale=V_SCALE)
    Bd.mimo_attn_decode_paged(glob, I["pq"], I["ppos"], O["kp"], O["vp"], I["table"], None, O["pout"],
                              ws=O["pws"], k_scale=K_SCALE, v_scale=V_SCALE)


def reset_caches(I, O):
    for c, c0 in (("rk", "rk0"), ("rv", "rv0"), ("kp", "kp0"), ("vp", "vp0")):
        O[c].copy_(I[c0])


CHECKED = ("rope", "out", "lse", "dq", "dk", "dv", "dsinks", "gout", "glse", "rk", "rv", "rout", "mout",
           "dout", "kp", "vp", "pout")


def test_whole_step_in_a_captured_graph():
    I = device_inputs(draw(0))
    G, E = outputs(I), outputs(I)
    rows = np.concatenate([np.arange(a, b) for a, b in zip(np.cumsum([0] + LENS_Q)[:-1], np.cumsum(LENS_Q))])
    reset_caches(I, G)
    step(I, G)                          # eager warm-up (loads the kernels' code objects)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(I, G)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        new = device_inputs(draw(r + 1))
        for name, t in new.items():
            if name not in ("ppos",):
                I[name].copy_(t)
        reset_caches(I, G)
        reset_caches(I, E)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(I, E)
        torch.cuda.synchronize()
        for name in CHECKED:
            a, b = G[name], E[name]
            same = torch.equal(a.view(torch.uint8), b.view(torch.uint8))
            if not same:
                say(f"  replay {r}: {name} differs from the eager call")
            assert same, name
        # packed rows are the only ones the packed call writes
        lr = torch.from_numpy(rows).cuda()
        assert torch.equal(G["lout"][lr].view(torch.int16), E["lout"][lr].view(torch.int16))
        assert torch.equal(G["llse"][:, lr], E["llse"][:, lr])
        assert torch.isfinite(E["out"].float()).all() and torch.isfinite(E["dq"].float()).all()
        say(f"  replay {r}: {len(CHECKED) + 2} outputs and caches equal the eager calls bit for bit")
