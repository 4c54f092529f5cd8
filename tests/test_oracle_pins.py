"""Pins for the fp64 oracle: values the pages print, closed forms, library
routines, invariants and a 40-digit brute force on tiny shapes.

None of these re-types the oracle: the brute force follows the Hugging Face
eager structure the techniques-map page quotes (full score matrix, mask, the
sink concatenated as an extra column, softmax, column dropped), the SDPA
checks go through torch's own attention routine, and the closed forms are
written from the mathematics of the special case.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
from global_attention_sinks_amd import inputs as gen

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def bf16(x):
    return gen.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def f64(bits):
    return gen.bf16_bits_to_f32(bits).astype(np.float64)


def rand_case(seed, nq, nk, hq, hkv, dqk, dv):
    g = np.random.SeedSequence(seed).spawn(3)
    return (gen.normal_bf16(g[0], (nq, hq, dqk)), gen.normal_bf16(g[1], (nk, hkv, dqk)),
            gen.normal_bf16(g[2], (nk, hkv, dv)))


# ---------------------------------------------------------------- RoPE pins

def test_cos_200000_matches_page():
    """Gaudi recipe page, Verified: exact cos(200000) = 0.9974.  The fastest
    frequency (pair 0) has angle == position for any base."""
    g = GOLDEN["cos_200000"]
    x = np.zeros((1, 1, 192), np.float32)
    x[0, 0, 0] = 1.0
    for base in (1e4, 1e7):
        y = oracle.rope_partial(bf16(x), np.array([200000]), base)
        assert round(y[0, 0, 0], g["decimals"]) == g["value"]
        assert abs(y[0, 0, 32] - math.sin(200000.0)) < 1e-12      # partner dim carries sin
        # what an fp32 angle product would have given is far off: the value is fp64
        assert abs(y[0, 0, 0] - 0.0) > 0.9


def test_rope_dim_and_split_from_page():
    """Techniques map, Partial RoPE: rope_dim = int(192*0.334) = 64, the first
    64 dims rotate and dims 64..191 pass through."""
    g = GOLDEN["rope_dim"]
    assert int(g["head_dim"] * g["partial_rotary_factor"]) == g["value"] == oracle.ROPE_DIM
    x = gen.normal_bf16(np.random.SeedSequence(5), (7, 3, 192))
    pos = np.array([1, 2, 3, 100, 1000, 77777, 500000])
    y = oracle.rope_partial(x, pos, 1e4)
    xf = f64(x)
    assert np.array_equal(y[..., 64:], xf[..., 64:])
    assert np.all(np.abs(y[..., :64] - xf[..., :64]).max(axis=-1) > 0)


def test_rope_identity_at_zero_and_norm_preserving():
    x = gen.normal_bf16(np.random.SeedSequence(6), (5, 4, 192))
    xf = f64(x)
    y0 = oracle.rope_partial(x, np.zeros(5, np.int64), 1e7)
    assert np.array_equal(y0, xf)
    y = oracle.rope_partial(x, np.array([3, 30, 3000, 300000, 524287]), 1e7)
    # each rotating pair (i, i+32) keeps its length
    n_in = xf[..., :32] ** 2 + xf[..., 32:64] ** 2
    n_out = y[..., :32] ** 2 + y[..., 32:64] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-13, atol=1e-13)


def test_rope_relative_position():
    """<rope(q,a), rope(k,b)> depends on a-b only (rotation group property)."""
    q = gen.normal_bf16(np.random.SeedSequence(7), (1, 1, 192))
    k = gen.normal_bf16(np.random.SeedSequence(8), (1, 1, 192))
    for base in (1e4, 1e7):
        d = []
        for a, b in [(10, 3), (1007, 1000), (400007, 400000)]:
            qa = oracle.rope_partial(q, np.array([a]), base)
            kb = oracle.rope_partial(k, np.array([b]), base)
            d.append(float((qa * kb).sum()))
        assert abs(d[0] - d[1]) < 1e-9 and abs(d[0] - d[2]) < 1e-8


# ---------------------------------------------------- brute force (mpmath)

mpmath.mp.dps = 40


def _mp_rope(vec, pos, base, R):
    half = R // 2
    out = list(vec)
    for i in range(half):
        th = mpmath.mpf(pos) * mpmath.power(mpmath.mpf(base), -mpmath.mpf(2 * i) / R)
        c, s = mpmath.cos(th), mpmath.sin(th)
        out[i] = vec[i] * c - vec[i + half] * s
        out[i + half] = vec[i + half] * c + vec[i] * s
    return out


def _mp_eager(q, k, v, qpos, kpos, sinks, window, base, R, scale, vscale):
    """HF eager structure: repeat_kv, scores, mask, cat sink column, softmax,
    drop the column, weights @ V, times the V scale."""
    nq, hq, _ = q.shape
    nk, hkv, _ = k.shape
    rep = hq // hkv
    out = np.zeros((nq, hq, v.shape[2]))
    for h in range(hq):
        g = h // rep                                   # repeat_kv: consecutive heads share
        for i in range(nq):
            qi = _mp_rope([mpmath.mpf(float(x)) for x in q[i, h]], int(qpos[i]), base, R)
            row = []
            for j in range(nk):
                kj = _mp_rope([mpmath.mpf(float(x)) for x in k[j, g]], int(kpos[j]), base, R)
                ok = kpos[j] <= qpos[i] and (window == 0 or qpos[i] - kpos[j] < window)
                row.append(mpmath.fsum(a * b for a, b in zip(qi, kj)) * scale if ok else None)
            cols = [x for x in row if x is not None]
            if sinks is not None:
                cols.append(mpmath.mpf(float(sinks[h])))
            if not cols:
                continue
            m = max(cols)
            z = mpmath.fsum(mpmath.exp(c - m) for c in cols)
            for d in range(v.shape[2]):
                acc = mpmath.fsum(mpmath.exp(row[j] - m) * mpmath.mpf(float(v[j, g, d]))
                                  for j in range(nk) if row[j] is not None)
                out[i, h, d] = float(acc / z * vscale)
    return out


@pytest.mark.parametrize("window,with_sink,hkv", [(0, False, 2), (3, True, 2), (1, True, 1),
                                                  (2, False, 1), (5, True, 2)])
def test_brute_force_tiny(window, with_sink, hkv):
    nq, hq, dqk, dv, R = 5, 4, 6, 4, 4
    qb, kb, vb = rand_case(11 + window, nq, nq, hq, hkv, dqk, dv)
    pos = np.array([3, 4, 5, 6, 7])
    sinks = np.array([0.3, -1.2, 2.0, 0.0]) if with_sink else None
    base = 1e4
    scale = 1.0 / math.sqrt(dqk)
    got = oracle.attention(qb, pos, kb, pos, vb, sinks=sinks, window=window, base=base,
                           softmax_scale=scale, v_scale=0.707, rope_dim=R)
    want = _mp_eager(f64(qb), f64(kb), f64(vb), pos, pos, sinks, window, base, R,
                     mpmath.mpf(1) / mpmath.sqrt(dqk), mpmath.mpf("0.707"))
    assert np.max(np.abs(got - want)) < 1e-12


# ------------------------------------------- library routine: torch SDPA

def _sdpa_reference(qr, kr, v, qpos, kpos, sinks, window, scale, vscale):
    """torch's scaled_dot_product_attention in float64 on CPU.  The sink is an
    extra key of zeros whose additive mask entry is the sink logit and whose
    value is zero."""
    nq, hq, _ = qr.shape
    nk, hkv, _ = kr.shape
    rep = hq // hkv
    Q = torch.from_numpy(qr).permute(1, 0, 2)                      # [H, nq, D]
    K = torch.from_numpy(kr).repeat_interleave(rep, dim=1).permute(1, 0, 2)
    V = torch.from_numpy(v).repeat_interleave(rep, dim=1).permute(1, 0, 2)
    qp = torch.from_numpy(qpos)[:, None]
    kp = torch.from_numpy(kpos)[None, :]
    vis = kp <= qp
    if window:
        vis &= (qp - kp) < window
    mask = torch.where(vis, 0.0, -math.inf).to(torch.float64).expand(hq, nq, nk)
    if sinks is not None:
        K = torch.cat([K, torch.zeros(hq, 1, K.shape[2], dtype=K.dtype)], dim=1)
        V = torch.cat([V, torch.zeros(hq, 1, V.shape[2], dtype=V.dtype)], dim=1)
        col = torch.from_numpy(np.asarray(sinks, np.float64))[:, None, None].expand(hq, nq, 1)
        mask = torch.cat([mask, col], dim=2)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    return (o * vscale).permute(1, 0, 2).numpy()


@pytest.mark.parametrize("window,with_sink,base,hkv", [(0, False, 1e7, 4), (128, True, 1e4, 8),
                                                       (16, True, 1e4, 8), (0, False, 1e4, 8)])
def test_against_torch_sdpa(window, with_sink, base, hkv):
    n = 300
    qb, kb, vb = rand_case(21 + window, n, n, 64, hkv, 192, 128)
    pos = np.arange(1000, 1000 + n, dtype=np.int64)
    sinks = gen.normal_f32(np.random.SeedSequence(3), (64,)).astype(np.float64) if with_sink else None
    got = oracle.attention(qb, pos, kb, pos, vb, sinks=sinks, window=window, base=base)
    qr = oracle.rope_partial(qb, pos, base)
    kr = oracle.rope_partial(kb, pos, base)
    want = _sdpa_reference(qr, kr, f64(vb), pos, pos, sinks, window, oracle.SOFTMAX_SCALE, 0.707)
    assert np.max(np.abs(got - want)) < 1e-12


# ------------------------------------------------------------ closed forms

def test_query_zero_closed_form_and_window_of_128():
    """q = 0: every score is 0, so o = v_scale * sum_j v_j / (n + e^sink) with
    n = number of visible keys; past the first 127 tokens n == 128, the HF
    window (miles page, 5.4 Notable quirks)."""
    W = GOLDEN["window_keys_total"]["value"]
    T, hq, hkv = 300, 8, 1
    _, kb, vb = rand_case(31, 1, T, hq, hkv, 192, 128)
    qb = np.zeros((T, hq, 192), np.uint16)
    sinks = np.linspace(-2, 2, hq)
    pos = np.arange(T, dtype=np.int64)
    got = oracle.attention(qb, pos, kb, pos, vb, sinks=sinks, window=W, base=1e4)
    vf = f64(vb)[:, 0, :]
    for t in (0, 1, 126, 127, 128, 200, 299):
        lo = max(0, t - W + 1)
        n = t - lo + 1
        assert n == min(t + 1, 128)
        for h in range(hq):
            want = 0.707 * vf[lo:t + 1].sum(0) / (n + math.exp(sinks[h]))
            assert np.max(np.abs(got[t, h] - want)) < 1e-13


def test_window_one_is_sigmoid_gate():
    """W = 1: each query sees only itself, o = v_scale * v_t * sigmoid(s_tt - sink)."""
    T = 9
    qb, kb, vb = rand_case(41, T, T, 4, 2, 192, 128)
    pos = np.arange(50, 50 + T, dtype=np.int64)
    sinks = np.array([0.5, -0.5, 3.0, -3.0])
    got = oracle.attention(qb, pos, kb, pos, vb, sinks=sinks, window=1, base=1e4)
    qr = oracle.rope_partial(qb, pos, 1e4)
    kr = oracle.rope_partial(kb, pos, 1e4)
    for t in range(T):
        for h in range(4):
            s = (qr[t, h] @ kr[t, h // 2]) / math.sqrt(192)
            gate = 1.0 / (1.0 + math.exp(sinks[h] - s))
            assert np.max(np.abs(got[t, h] - 0.707 * f64(vb)[t, h // 2] * gate)) < 1e-13


def test_window_at_least_T_is_full_causal():
    T = 64
    qb, kb, vb = rand_case(51, T, T, 8, 2, 192, 128)
    pos = np.arange(T, dtype=np.int64)
    a = oracle.attention(qb, pos, kb, pos, vb, window=T, base=1e4)
    b = oracle.attention(qb, pos, kb, pos, vb, window=0, base=1e4)
    c = oracle.attention(qb, pos, kb, pos, vb, window=10 * T, base=1e4)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_sink_limits():
    """sink -> -inf is plain causal softmax; sink -> +inf drives o to 0."""
    T = 40
    qb, kb, vb = rand_case(61, T, T, 8, 1, 192, 128)
    pos = np.arange(T, dtype=np.int64)
    plain = oracle.attention(qb, pos, kb, pos, vb, window=16, base=1e4)
    neg = oracle.attention(qb, pos, kb, pos, vb, sinks=np.full(8, -1e300), window=16, base=1e4)
    assert np.max(np.abs(plain - neg)) == 0.0
    pos_inf, ps = oracle.attention(qb, pos, kb, pos, vb, sinks=np.full(8, 800.0), window=16,
                                   base=1e4, want_psink=True)
    assert np.max(np.abs(pos_inf)) < 1e-300 and np.all(ps == 1.0)


def test_row_sum_and_convexity():
    """p_sink + sum_j p_j = 1 and o / v_scale lies in (1 - p_sink) * [min v, max v]."""
    T = 200
    qb, kb, vb = rand_case(71, T, T, 16, 2, 192, 128)
    pos = np.arange(T, dtype=np.int64)
    sinks = np.linspace(-3, 3, 16)
    out, lse, ps = oracle.attention(qb, pos, kb, pos, vb, sinks=sinks, window=128, base=1e4,
                                    want_lse=True, want_psink=True)
    vf = f64(vb)
    qr = oracle.rope_partial(qb, pos, 1e4)
    kr = oracle.rope_partial(kb, pos, 1e4)
    for t in (0, 5, 127, 128, 199):
        lo = max(0, t - 127)
        for h in (0, 7, 15):
            g = h // 8
            s = kr[lo:t + 1, g] @ qr[t, h] / math.sqrt(192)
            p = np.exp(s - lse[t, h])
            assert abs(p.sum() + ps[t, h] - 1.0) < 1e-12
            assert abs(ps[t, h] - math.exp(sinks[h] - lse[t, h])) < 1e-12
            w = 1.0 - ps[t, h]
            lo_v = vf[lo:t + 1, g].min(0) * w
            hi_v = vf[lo:t + 1, g].max(0) * w
            o = out[t, h] / 0.707
            assert np.all(o >= lo_v - 1e-12) and np.all(o <= hi_v + 1e-12)


def test_gqa_equals_expanded_mha():
    """repeat_kv: running GQA equals running MHA on K/V with each KV head
    repeated for its consecutive query heads."""
    T, hq, hkv = 50, 16, 4
    qb, kb, vb = rand_case(81, T, T, hq, hkv, 192, 128)
    pos = np.arange(T, dtype=np.int64)
    a = oracle.attention(qb, pos, kb, pos, vb, window=0, base=1e7)
    kx = np.repeat(kb, hq // hkv, axis=1)
    vx = np.repeat(vb, hq // hkv, axis=1)
    b = oracle.attention(qb, pos, kx, pos, vx, window=0, base=1e7)
    assert np.array_equal(a, b)
    # and a different grouping (h mod Hkv) would not agree
    kw = np.tile(kb, (1, hq // hkv, 1))
    vw = np.tile(vb, (1, hq // hkv, 1))
    c = oracle.attention(qb, pos, kw, pos, vw, window=0, base=1e7)
    assert np.max(np.abs(a - c)) > 1e-3


def test_position_shift_invariance():
    T = 80
    qb, kb, vb = rand_case(91, T, T, 8, 1, 192, 128)
    sinks = np.linspace(-1, 1, 8)
    p0 = np.arange(T, dtype=np.int64)
    a = oracle.attention(qb, p0, kb, p0, vb, sinks=sinks, window=32, base=1e4)
    b = oracle.attention(qb, p0 + 123456, kb, p0 + 123456, vb, sinks=sinks, window=32, base=1e4)
    assert np.max(np.abs(a - b)) < 1e-9


def test_chunked_global_prefill_equals_whole():
    B, T = 1, 96
    d = gen.prefill_inputs(B, T, 8, 2, seed=7, with_sinks=False)
    whole = oracle.prefill_global(d["q"], d["k"], d["v"], base=1e7)
    parts = []
    for c in range(3):
        qc = d["q"][:, c * 32:(c + 1) * 32]
        hi = (c + 1) * 32
        parts.append(oracle.prefill_global(qc, d["k"][:, :hi], d["v"][:, :hi], q_pos0=c * 32, base=1e7))
    assert np.array_equal(np.concatenate(parts, axis=1), whole)


def test_varlen_chunk_continuation_equals_whole_sequence():
    """A chunk that continues a sequence, given only the window-1 keys before it
    (sliding) or its whole prefix (global), reproduces the whole prefill's rows."""
    T, lo = 300, 200
    d = gen.prefill_inputs(1, T, 8, 2, seed=21, with_sinks=True)
    whole_s = oracle.prefill_swa(d["q"], d["k"], d["v"], d["sinks"], window=128, base=1e4)[0]
    whole_g = oracle.prefill_global(d["q"], d["k"], d["v"], base=1e7)[0]
    k0 = lo - 127
    cu_q = np.array([0, T - lo], np.int32)
    got_s = oracle.prefill_varlen(d["q"][0, lo:], d["k"][0, k0:], d["v"][0, k0:], cu_q,
                                  np.array([0, T - k0], np.int32), k_pos0=np.array([k0]), sinks=d["sinks"],
                                  window=128, base=1e4)
    assert np.array_equal(got_s, whole_s[lo:])
    got_g = oracle.prefill_varlen(d["q"][0, lo:], d["k"][0], d["v"][0], cu_q, np.array([0, T], np.int32),
                                  window=0, base=1e7)
    assert np.array_equal(got_g, whole_g[lo:])
    # one key fewer than the window needs changes the first row of the chunk
    short = oracle.prefill_varlen(d["q"][0, lo:], d["k"][0, k0 + 1:], d["v"][0, k0 + 1:], cu_q,
                                  np.array([0, T - k0 - 1], np.int32), k_pos0=np.array([k0 + 1]),
                                  sinks=d["sinks"], window=128, base=1e4)
    assert np.max(np.abs(short[0] - whole_s[lo])) > 1e-6
    assert np.array_equal(short[1:], whole_s[lo + 1:])


def test_varlen_packing_equals_separate_sequences():
    lens = [37, 1, 0, 130]
    seqs = [gen.prefill_inputs(1, L, 8, 1, seed=30 + i, with_sinks=False) for i, L in enumerate(lens)]
    sinks = np.linspace(-2, 2, 8).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = np.concatenate([s["q"][0] for s in seqs])
    k = np.concatenate([s["k"][0] for s in seqs])
    v = np.concatenate([s["v"][0] for s in seqs])
    pos0 = np.array([0, 5, 9, 1000], np.int64)
    out, lse = oracle.prefill_varlen(q, k, v, cu, cu, k_pos0=pos0, sinks=sinks, window=128, base=1e4,
                                     want_lse=True)
    for i, s in enumerate(seqs):
        if lens[i] == 0:
            continue
        ref, rl = oracle.prefill_swa(s["q"], s["k"], s["v"], sinks, pos0=int(pos0[i]), window=128, base=1e4,
                                     want_lse=True)
        assert np.array_equal(out[cu[i]:cu[i + 1]], ref[0])
        assert np.array_equal(lse[:, cu[i]:cu[i + 1]], rl[0].T)


def test_decode_cache_rule_matches_prefill_rows():
    """A decode query over a ring cache that holds the rotated keys sees exactly
    the keys the prefill row sees: checked on exactly representable values."""
    T, cap, W = 300, 128, 128
    d = gen.prefill_inputs(1, T, 8, 1, seed=9, with_sinks=True)
    # keys with no rotary part, so their rotated value is exact in bf16
    k = d["k"].copy()
    k[..., :64] = 0
    pref = oracle.prefill_swa(d["q"], k, d["v"], d["sinks"], window=W, base=1e4)
    for p in (5, 127, 128, 250, 299):
        kc = np.full((1, cap, 1, 192), gen.BF16_NAN, np.uint16)
        vc = np.full((1, cap, 1, 128), gen.BF16_NAN, np.uint16)
        for t in range(max(0, p - W + 1), p + 1):
            kc[0, t % cap] = k[0, t]
            vc[0, t % cap] = d["v"][0, t]
        o = oracle.decode(d["q"][0, p][None], np.array([p]), kc, vc, sinks=d["sinks"], window=W, base=1e4)
        assert np.max(np.abs(o[0] - pref[0, p])) < 1e-13


@pytest.mark.parametrize("window,cap", [(128, 135), (0, 400)])
def test_decode_multi_matches_prefill_rows(window, cap):
    """n_q draft tokens verified together over a cache that holds them see exactly
    what their prefill rows see (exactly representable keys, as above); a token
    at a negative position gets zeros."""
    T, nq = 300, 8
    d = gen.prefill_inputs(1, T, 8, 1, seed=10, with_sinks=window > 0)
    k = d["k"].copy()
    k[..., :64] = 0
    if window:
        pref = oracle.prefill_swa(d["q"], k, d["v"], d["sinks"], window=window, base=1e4)[0]
    else:
        pref = oracle.prefill_global(d["q"], k, d["v"], base=1e7)[0]
    for p in (3, 7, 130, 299):
        kc = np.full((1, cap, 1, 192), gen.BF16_NAN, np.uint16)
        vc = np.full((1, cap, 1, 128), gen.BF16_NAN, np.uint16)
        for t in range(max(0, p - cap + 1), p + 1):
            kc[0, t % cap] = k[0, t]
            vc[0, t % cap] = d["v"][0, t]
        q = np.zeros((1, nq, 8, 192), np.uint16)
        for i in range(nq):
            q[0, i] = d["q"][0, max(0, p - nq + 1 + i)]
        o = oracle.decode_multi(q, np.array([p]), kc, vc, sinks=d["sinks"], window=window,
                                base=1e4 if window else 1e7)[0]
        for i in range(nq):
            t = p - nq + 1 + i
            if t < 0:
                assert np.all(o[i] == 0.0)
            else:
                assert np.max(np.abs(o[i] - pref[t])) < 1e-13


# ---------------------------------------------------------------- backward

def _torch_eager_rows(q, k, v, qpos, kpos, sinks, window, base, R, scale, vscale):
    """The eager structure in float64 torch ops (RoPE, repeat_kv, scores, mask,
    sink column, softmax, column dropped, @ V, V scale); differentiable."""
    half = R // 2
    inv = torch.tensor([base ** (-(2 * i) / R) for i in range(half)], dtype=torch.float64)

    def rope(x, pos):
        ang = torch.from_numpy(pos.astype(np.float64))[:, None] * inv[None, :]
        c, s_ = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
        a, b = x[..., :half], x[..., half:R]
        return torch.cat([a * c - b * s_, b * c + a * s_, x[..., R:]], dim=-1)

    hq, hkv = q.shape[1], k.shape[1]
    qr, kr = rope(q, qpos), rope(k, kpos)
    kr = kr.repeat_interleave(hq // hkv, dim=1)
    vv = v.repeat_interleave(hq // hkv, dim=1)
    sc = torch.einsum("ihd,jhd->hij", qr, kr) * scale
    qp, kp = torch.from_numpy(qpos)[:, None], torch.from_numpy(kpos)[None, :]
    vis = kp <= qp
    if window:
        vis &= (qp - kp) < window
    sc = sc.masked_fill(~vis[None], -math.inf)
    if sinks is not None:
        sc = torch.cat([sc, sinks[:, None, None].expand(hq, q.shape[0], 1)], dim=2)
    p = torch.softmax(sc, dim=2)[:, :, :k.shape[0]]
    return torch.einsum("hij,jhd->ihd", p, vv) * vscale


@pytest.mark.parametrize("window,with_sink,hkv", [(0, False, 2), (5, True, 2), (1, True, 1), (16, True, 4)])
def test_backward_matches_autograd(window, with_sink, hkv):
    """The oracle's chain-rule gradients against torch autograd (float64) through
    the eager structure."""
    n, hq, dqk, dv, R = 24, 8, 12, 8, 8
    qb, kb, vb = rand_case(51 + window, n, n, hq, hkv, dqk, dv)
    dob = gen.normal_bf16(np.random.SeedSequence(52 + window), (n, hq, dv))
    pos = np.arange(500, 500 + n, dtype=np.int64)
    sinks = np.linspace(-1.5, 2.0, hq) if with_sink else None
    scale = 1.0 / math.sqrt(dqk)
    got = oracle.attention_backward(qb, pos, kb, pos, vb, dob, sinks=sinks, window=window, base=1e4,
                                    softmax_scale=scale, v_scale=0.707, rope_dim=R)
    Q = torch.tensor(f64(qb), requires_grad=True)
    K = torch.tensor(f64(kb), requires_grad=True)
    V = torch.tensor(f64(vb), requires_grad=True)
    Sk = torch.tensor(sinks, requires_grad=True) if with_sink else None
    out = _torch_eager_rows(Q, K, V, pos, pos, Sk, window, 1e4, R, scale, 0.707)
    out.backward(torch.tensor(f64(dob)))
    for a, b in ((got[0], Q.grad), (got[1], K.grad), (got[2], V.grad)):
        assert np.max(np.abs(a - b.numpy())) < 1e-12
    if with_sink:
        assert np.max(np.abs(got[3] - Sk.grad.numpy())) < 1e-12
    else:
        assert got[3] is None


def test_backward_window_one_closed_form():
    """W = 1: o_t = 0.707 g_t v_t with g_t = sigmoid(s_tt - sink), so
    dv_t = 0.707 g_t dO_t and d sink = -sum_t 0.707 g_t (1 - g_t) <dO_t, v_t>."""
    n = 40
    qb, kb, vb = rand_case(61, n, n, 4, 1, 192, 128)
    dob = gen.normal_bf16(np.random.SeedSequence(62), (n, 4, 128))
    pos = np.arange(n, dtype=np.int64)
    sinks = np.array([0.5, -0.5, 1.5, 0.0])
    _, _, dv, ds = oracle.attention_backward(qb, pos, kb, pos, vb, dob, sinks=sinks, window=1, base=1e4)
    qr, kr = oracle.rope_partial(qb, pos, 1e4), oracle.rope_partial(kb, pos, 1e4)
    s_tt = np.einsum("thd,td->th", qr, kr[:, 0]) * oracle.SOFTMAX_SCALE
    g = 1.0 / (1.0 + np.exp(-(s_tt - sinks[None, :])))
    dO, v = f64(dob), f64(vb)[:, 0]
    assert np.max(np.abs(dv[:, 0] - 0.707 * np.einsum("th,thd->td", g, dO))) < 1e-12
    want = -np.sum(0.707 * g * (1 - g) * np.einsum("thd,td->th", dO, v), axis=0)
    assert np.max(np.abs(ds - want)) < 1e-12


def test_backward_position_shift_invariance():
    """Shifting every position changes no score, so no gradient of the unrotated
    inputs either."""
    n = 60
    qb, kb, vb = rand_case(71, n, n, 8, 1, 192, 128)
    dob = gen.normal_bf16(np.random.SeedSequence(72), (n, 8, 128))
    p0 = np.arange(n, dtype=np.int64)
    sinks = np.linspace(-1, 1, 8)
    a = oracle.attention_backward(qb, p0, kb, p0, vb, dob, sinks=sinks, window=16, base=1e4)
    b = oracle.attention_backward(qb, p0 + 99999, kb, p0 + 99999, vb, dob, sinks=sinks, window=16, base=1e4)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) < 1e-9


# ---------------------------------------------------------------- fp8 e4m3 and paged caches

def test_e4m3_decode_closed_forms_and_library():
    """OCP e4m3: exponent bias 7, 3 mantissa bits, subnormals below 2^-6, 448 the
    largest value, 0x7F NaN; and every code against torch's float8_e4m3fn."""
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3F: 1.875,
             0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in known.items():
        assert oracle.e4m3_to_f64([c])[0] == v, hex(c)
    assert np.isnan(oracle.e4m3_to_f64([0x7F, 0xFF])).all()
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(oracle.e4m3_to_f64(codes), lib, equal_nan=True)


def test_e4m3_round_nearest_even_saturating():
    # midpoints go to the even code; beyond 448 saturates; subnormal midpoints too
    assert list(oracle.e4m3_round([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 500.0, -1000.0])) == \
        [0x38, 0x3A, 0x00, 0x02, 0x7E, 0xFE]
    x = np.random.default_rng(1).standard_normal(200000) * 60
    x = x[np.abs(x) < 448]
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(oracle.e4m3_to_f64(oracle.e4m3_round(x)), lib)


@pytest.mark.parametrize("window,nq", [(0, 1), (0, 4), (128, 8)])
def test_paged_decode_equals_contiguous_cache(window, nq):
    """The same tokens in shuffled pool blocks or in a per-sequence cache give the
    same result (bf16 pools)."""
    S, bs = 3, 32
    pos = np.array([40, 150, 5], np.int64)
    d = gen.paged_decode_inputs(S, nq, bs, 8, 2, seed=40, window=window, pos=pos, with_sinks=window > 0)
    cap = 160 if window == 0 else window + nq - 1
    kc = np.full((S, cap, 2, 192), gen.BF16_NAN, np.uint16)
    vc = np.full((S, cap, 2, 128), gen.BF16_NAN, np.uint16)
    for s in range(S):
        p = int(pos[s])
        lo = max(0, p - (nq - 1) - window + 1) if window else 0
        for t in range(lo, p + 1):
            kc[s, t % cap] = d["k_pool"][d["table"][s, t // bs], t % bs]
            vc[s, t % cap] = d["v_pool"][d["table"][s, t // bs], t % bs]
    base = 1e4 if window else 1e7
    a = oracle.decode_paged(d["q"], pos, d["k_pool"], d["v_pool"], d["table"], block_size=bs, sinks=d["sinks"],
                            window=window, base=base)
    b = oracle.decode_multi(d["q"], pos, kc, vc, sinks=d["sinks"], window=window, base=base)
    assert np.array_equal(a, b)


def test_fp8_paged_decode_equals_bf16_of_the_values():
    """fp8 codes with power-of-two scales hold values bf16 represents exactly:
    the fp8 paged decode equals the bf16 paged decode of those values."""
    S, bs, nq = 2, 32, 2
    pos = np.array([70, 33], np.int64)
    ks, vs = 2.0 ** -3, 2.0 ** 2
    d = gen.paged_decode_inputs(S, nq, bs, 8, 2, seed=41, window=0, pos=pos, with_sinks=False,
                                kv_dtype="fp8", k_scale=ks, v_scale=vs)
    kval = oracle.e4m3_to_f64(d["k_pool"]) * ks
    vval = oracle.e4m3_to_f64(d["v_pool"]) * vs
    kb = gen.f32_to_bf16_bits(kval.astype(np.float32))
    vb = gen.f32_to_bf16_bits(vval.astype(np.float32))
    assert np.array_equal(gen.bf16_bits_to_f32(kb).astype(np.float64), kval, equal_nan=True)
    a = oracle.decode_paged(d["q"], pos, d["k_pool"], d["v_pool"], d["table"], block_size=bs, kv_dtype="fp8",
                            k_scale=ks, v_scale=vs, window=0, base=1e7)
    b = oracle.decode_paged(d["q"], pos, kb, vb, d["table"], block_size=bs, window=0, base=1e7)
    assert np.max(np.abs(a - b)) < 1e-12


def test_input_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 65504.0], np.float32)
    b = gen.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 -> 1+2^-6
    assert list(gen.bf16_bits_to_f32(b)[:3]) == [1.0, 1.0, 1.015625]
    assert np.allclose(gen.bf16_bits_to_f32(b), x, rtol=2 ** -8)


# ------------------------------------- bf16 operands: rounded rows and their bound

def _scaled_case(seed, nq, nk, hq, hkv, qmul, kmul):
    qb, kb, vb = rand_case(seed, nq, nk, hq, hkv, 192, 128)
    return bf16(f64(qb) * qmul), bf16(f64(kb) * kmul), vb


def _round_rotated(x):
    """The first 64 (rotated) dims through torch's bfloat16 cast; the rest unchanged."""
    y = x.copy()
    y[..., :64] = torch.from_numpy(np.ascontiguousarray(x[..., :64])).to(torch.bfloat16).to(torch.float64).numpy()
    return y


@pytest.mark.parametrize("window,with_sink", [(0, False), (16, True)])
def test_operand_rounding_rows_match_sdpa_on_rounded_operands(window, with_sink):
    """out_rounded equals torch SDPA over rope(q), rope(k) whose rotated dims went
    through torch's own bf16 cast; at position 0 (no rotation) nothing is rounded
    and out_rounded is the exact row."""
    nq = nk = 40
    qb, kb, vb = _scaled_case(71 + window, nq, nk, 4, 2, 2.0, 4.0)
    sinks = np.array([0.5, -1.0, 2.0, 0.0]) if with_sink else None
    pos = np.arange(90000, 90000 + nk, dtype=np.int64)
    got, bound = oracle.operand_rounding(qb, pos, kb, pos, vb, sinks=sinks, window=window, base=1e7)
    qr = _round_rotated(oracle.rope_partial(qb, pos, 1e7))
    kr = _round_rotated(oracle.rope_partial(kb, pos, 1e7))
    want = _sdpa_reference(qr, kr, f64(vb), pos, pos, sinks, window, oracle.SOFTMAX_SCALE, 0.707)
    assert np.max(np.abs(got - want)) < 1e-12
    exact = oracle.attention(qb, pos, kb, pos, vb, sinks=sinks, window=window, base=1e7)
    assert np.max(np.abs(got - exact)) > 1e-4          # the rounding does move these rows
    assert np.all(np.abs(got - exact) <= bound)
    z = np.zeros(nk, np.int64)                           # one position: no rotation
    got0, _ = oracle.operand_rounding(qb, z, kb, z, vb, sinks=sinks, window=0, base=1e7)
    assert np.max(np.abs(got0 - oracle.attention(qb, z, kb, z, vb, sinks=sinks, window=0, base=1e7))) < 1e-13


@pytest.mark.parametrize("window,with_sink", [(0, False), (16, True)])
def test_operand_rounding_bound_holds_for_adversarial_perturbations(window, with_sink):
    """Brute force over perturbations of the rotated operands within bf16's unit
    roundoff 2^-8 (torch SDPA on the perturbed operands): random ones stay within
    the bound everywhere, and one aimed at a chosen output element (every key's
    score pushed by half the per-score budget, each in the direction that moves
    that element up) reaches a good part of its bound, so the bound is not vacuous."""
    nq, nk, hq, hkv = 8, 48, 4, 2
    qb, kb, vb = _scaled_case(91 + window, nq, nk, hq, hkv, 2.0, 4.0)
    sinks = np.array([1.0, -0.5, 0.0, 2.5]) if with_sink else None
    pos = np.arange(200000, 200000 + nk, dtype=np.int64)
    qpos = pos[nk - nq:]
    q_rows = qb[:nq]
    u = 2.0 ** -8
    base, scale = 1e7, oracle.SOFTMAX_SCALE
    exact = oracle.attention(q_rows, qpos, kb, pos, vb, sinks=sinks, window=window, base=base)
    _, bound = oracle.operand_rounding(q_rows, qpos, kb, pos, vb, sinks=sinks, window=window, base=base)
    qr = oracle.rope_partial(q_rows, qpos, base)
    kr = oracle.rope_partial(kb, pos, base)
    v = f64(vb)
    rng = np.random.default_rng(5)
    for _ in range(20):
        eq = rng.uniform(-u, u, qr.shape)
        ek = rng.uniform(-u, u, kr.shape)
        eq[..., 64:] = 0
        ek[..., 64:] = 0
        o = _sdpa_reference(qr * (1 + eq), kr * (1 + ek), v, qpos, pos, sinks, window, scale, 0.707)
        assert np.all(np.abs(o - exact) <= bound)
    # aimed: row r, head h, dim d; keys of KV head g get k_i (1 + u sign(q_i k_i) sigma_j)
    r, h, d = nq - 1, 3, 17
    g = h // (hq // hkv)
    s = scale * np.einsum("d,jd->j", qr[r, h], kr[:, g])
    vis = (pos <= qpos[r]) & ((qpos[r] - pos < window) if window else True)
    s = np.where(vis, s, -np.inf)
    m = max(s.max(), sinks[h] if with_sink else -np.inf)
    p = np.exp(s - m) / (np.exp(s - m).sum() + (np.exp(sinks[h] - m) if with_sink else 0.0))
    sigma = np.sign(p * (0.707 * v[:, g, d] - exact[r, h, d]))
    ek = np.zeros_like(kr)
    ek[:, g, :64] = u * np.sign(qr[r, h, None, :64] * kr[:, g, :64]) * sigma[:, None]
    o = _sdpa_reference(qr, kr * (1 + ek), v, qpos, pos, sinks, window, scale, 0.707)
    moved = o[r, h, d] - exact[r, h, d]
    assert 0 < moved <= bound[r, h, d]
    assert moved >= 0.1 * bound[r, h, d]
