"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch.

None of these calls reaches a kernel launch: each one fails validation first
(the pointer values are never dereferenced on the host)."""
import ctypes
import os
import re

import pytest

from global_attention_sinks_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mimo_attn.h")

OK, INVAL, UNSUP, WS, HIPERR = 0, 1, 2, 3, 4
FAKE = ctypes.c_void_p(0x10000)   # a non-NULL device address, never touched on the host


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from global_attention_sinks_amd import build
        build.build()
    return B.load_library()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mimo_status|size_t|const char \*)\s*(mimo_\w+)\s*\(", text, re.M)))


def test_header_lists_the_five_entry_points():
    fns = header_functions()
    for name in ("mimo_attn_prefill_swa", "mimo_attn_prefill_global", "mimo_attn_decode",
                 "mimo_rope_partial", "mimo_kv_ring_append"):
        assert name in fns


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_peak_loop_library_exports_its_header():
    """include/mimo_peaks.h declares the on-box peak loops of libmimo_peaks.so (measurement
    only): the library loads and exports each of them (none is called here)."""
    text = open(os.path.join(ROOT, "include", "mimo_peaks.h")).read()
    names = sorted(set(re.findall(r"^\s*int\s+(mimo_peak_\w+)\s*\(", text, re.M)))
    assert len(names) == 5, names
    if not os.path.exists(B.PEAKS_PATH):
        from global_attention_sinks_amd import build
        build.build()
    peaks = B.load_peaks()
    for name in names:
        assert hasattr(peaks, name), name


def cfg_swa(**kw):
    c = B.swa_cfg()
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def cfg_glob(**kw):
    c = B.global_cfg()
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def err(lib):
    return lib.mimo_last_error().decode()


def swa(lib, cfg, q=FAKE, k=FAKE, v=FAKE, sinks=FAKE, Bn=1, T=16, pos0=0, out=FAKE):
    return lib.mimo_attn_prefill_swa(ctypes.byref(cfg), q, k, v, sinks, Bn, T, pos0, out, None, None)


def glob(lib, cfg, Bn=1, Tq=16, Tk=16, q_pos0=0, q=FAKE, out=FAKE, ws=None, ws_bytes=0):
    return lib.mimo_attn_prefill_global(ctypes.byref(cfg), q, FAKE, FAKE, Bn, Tq, Tk, q_pos0, out, None, ws,
                                        ws_bytes, None)


def test_null_cfg(lib):
    assert lib.mimo_attn_prefill_swa(None, FAKE, FAKE, FAKE, FAKE, 1, 1, 0, FAKE, None, None) == INVAL
    assert "cfg" in err(lib)


@pytest.mark.parametrize("field,value,code", [
    ("num_q_heads", 0, INVAL), ("num_kv_heads", -1, INVAL), ("num_kv_heads", 7, INVAL),
    ("head_dim_qk", 128, UNSUP), ("head_dim_v", 192, UNSUP), ("rope_dim", 32, UNSUP),
    ("rope_base", 0.5, INVAL), ("rope_base", float("inf"), INVAL),
    ("softmax_scale", 0.0, INVAL), ("softmax_scale", float("nan"), INVAL),
    ("v_scale", float("inf"), INVAL), ("window", -1, INVAL), ("window", 0, INVAL),
])
def test_bad_cfg_swa(lib, field, value, code):
    assert swa(lib, cfg_swa(**{field: value})) == code
    assert err(lib)


def test_group_size_support(lib):
    # 64 q heads over 32 KV heads: group 2 is not a multiple of 4
    assert swa(lib, cfg_swa(num_kv_heads=32)) == UNSUP
    assert "multiple of 4" in err(lib)


def test_null_pointers_and_sizes(lib):
    c = cfg_swa()
    assert swa(lib, c, q=None) == INVAL
    assert swa(lib, c, out=None) == INVAL
    assert swa(lib, c, T=-1) == INVAL
    assert swa(lib, c, pos0=-5) == INVAL
    # empty work is valid and enqueues nothing, NULL data included
    assert swa(lib, c, q=None, k=None, v=None, out=None, T=0) == OK
    assert swa(lib, c, Bn=0) == OK


def test_global_prefill_contract(lib):
    assert glob(lib, cfg_glob(window=128)) == INVAL
    assert glob(lib, cfg_glob(), Tq=16, Tk=17) == INVAL
    assert "q_pos0 + Tq" in err(lib)
    assert glob(lib, cfg_glob(), Tq=16, Tk=48, q_pos0=-32) == INVAL
    assert glob(lib, cfg_glob(), Tq=0, Tk=0, q=None, out=None) == OK


def test_global_prefill_null_workspace_is_the_plain_call(lib):
    """The boundary's global prefill is q, k, v in and out out (one query chunk
    against its prefix).  The tile-image workspace is an optional extra: ws = NULL
    is accepted at every size (the attention kernel then stages each tile itself;
    tests/test_gpu_parity.py and tests/test_gpu_fullsize.py run it against the
    oracle as the "staged" cases), ws_bytes is not looked at without a ws, and the
    only workspace error is a non-NULL ws smaller than the size query."""
    for ws_bytes in (0, 5):
        assert glob(lib, cfg_glob(), Tq=16, Tk=17, ws=None, ws_bytes=ws_bytes) == INVAL
        assert "q_pos0 + Tq" in err(lib)          # the error is the real one, never the workspace
        assert glob(lib, cfg_glob(), Tq=0, Tk=0, q=None, out=None, ws=None, ws_bytes=ws_bytes) == OK
    need = lib.mimo_attn_prefill_workspace_size(ctypes.byref(cfg_glob()), 1, 16)
    assert glob(lib, cfg_glob(), ws=FAKE, ws_bytes=need - 1) == WS
    # the sliding prefill's sinks may be NULL (no sink column), never required
    assert swa(lib, cfg_swa(), sinks=None, T=0) == OK
    assert swa(lib, cfg_swa(), sinks=None, T=-1) == INVAL and "sink" not in err(lib)


def varlen(lib, cfg, Bn=2, max_q=64, total_q=128, q=FAKE, cu_q=FAKE, cu_k=FAKE, total_k=256, ws=None, ws_bytes=0):
    return lib.mimo_attn_prefill_varlen(ctypes.byref(cfg), q, FAKE, FAKE, None, Bn, cu_q, cu_k, None, max_q,
                                        total_q, total_k, FAKE, None, ws, ws_bytes, None)


def test_varlen_prefill_contract(lib):
    assert varlen(lib, cfg_swa(), Bn=-1) == INVAL
    assert varlen(lib, cfg_swa(), max_q=-1) == INVAL
    assert varlen(lib, cfg_swa(), max_q=200, total_q=100) == INVAL   # a sequence longer than the pack
    assert "total_q" in err(lib)
    assert varlen(lib, cfg_swa(), cu_q=None) == INVAL
    assert varlen(lib, cfg_glob(), q=None) == INVAL
    assert varlen(lib, cfg_swa(num_q_heads=8, num_kv_heads=4)) == UNSUP     # group of 2
    # nothing to do is valid with NULL data
    assert varlen(lib, cfg_swa(), Bn=0, q=None, cu_q=None, cu_k=None) == OK
    assert varlen(lib, cfg_glob(), max_q=0, total_q=0, q=None) == OK


# One image per 64-key tile and KV head: K rows of 192 + 8 pad elements, then V^T rows
# of 64 + 8, all bf16, plus one fp32 key norm; a packed call may start each sequence
# on a fresh tile.
IMAGE_BYTES = (64 * 200 + 128 * 72) * 2 + 4


def test_prefill_workspace_size(lib):
    size = lambda cfg, b, tk: lib.mimo_attn_prefill_workspace_size(ctypes.byref(cfg), b, tk)
    assert IMAGE_BYTES == 44036
    assert size(cfg_glob(), 1, 32768) == (512 + 1) * 4 * IMAGE_BYTES
    assert size(cfg_glob(), 4, 4 * 1000) == (63 + 4) * 4 * IMAGE_BYTES
    # a dense batch of B sequences of Tk keys fits in the size for B * Tk keys
    for b, tk in ((1, 1), (3, 63), (3, 65), (2, 8192), (5, 777)):
        assert size(cfg_glob(), b, b * tk) >= b * -(-tk // 64) * 4 * IMAGE_BYTES
    assert size(cfg_swa(), 1, 32768) == 0                                  # sliding layers stage in-kernel
    assert size(cfg_glob(num_q_heads=16), 1, 4096) == 0                     # GQA group 4
    assert size(cfg_glob(num_kv_heads=7), 1, 4096) == 0                     # invalid cfg
    assert size(cfg_glob(), 0, 4096) == 0 and size(cfg_glob(), 1, 0) == 0


def test_prefill_workspace_too_small(lib):
    need = lib.mimo_attn_prefill_workspace_size(ctypes.byref(cfg_glob()), 1, 16)
    assert glob(lib, cfg_glob(), ws=FAKE, ws_bytes=need - 1) == WS
    assert "workspace" in err(lib)
    assert varlen(lib, cfg_glob(), total_k=256, ws=FAKE, ws_bytes=4096) == WS
    assert varlen(lib, cfg_glob(), total_k=-1) == INVAL


def dec(lib, cfg, S=4, cap=128, ws=FAKE, ws_bytes=1 << 30, q=FAKE):
    return lib.mimo_attn_decode(ctypes.byref(cfg), S, q, FAKE, FAKE, FAKE, cap, None, FAKE, ws, ws_bytes, None)


def test_decode_contract(lib):
    assert dec(lib, cfg_swa(), cap=64) == INVAL          # ring shorter than the window
    assert "cap" in err(lib)
    assert dec(lib, cfg_swa(), S=-1) == INVAL
    assert dec(lib, cfg_swa(num_kv_heads=2), cap=128) == UNSUP   # group 32 > 16
    assert dec(lib, cfg_swa(num_q_heads=64, num_kv_heads=16), cap=128) == UNSUP   # 16 KV heads
    assert dec(lib, cfg_glob(), cap=(1 << 30) + 1) == UNSUP
    assert dec(lib, cfg_glob(), q=None) == INVAL
    assert dec(lib, cfg_glob(), S=0, q=None) == OK


def test_decode_workspace(lib):
    g = cfg_glob()
    need = lib.mimo_attn_decode_workspace_size(ctypes.byref(g), 16, 131072)
    # partials (max, sum, 128 outputs) in fp32 for up to 1024/Hkv workgroup pieces
    # plus one per sequence, for every query head; then the plan: an int64 step
    # start per sequence (+1 total), three int32 per sequence and one per workgroup
    def expect(S, hkv):
        return (1024 // hkv + S) * 64 * (128 + 2) * 4 + (S + 1) * 8 + 3 * S * 4 + (1024 // hkv) * 4
    assert need == expect(16, 4)
    # independent of the cache length
    assert lib.mimo_attn_decode_workspace_size(ctypes.byref(g), 16, 4096) == need
    assert lib.mimo_attn_decode_workspace_size(ctypes.byref(cfg_swa()), 64, 128) == expect(64, 8)
    assert dec(lib, g, S=16, cap=131072, ws=None, ws_bytes=0) == WS
    assert dec(lib, g, S=16, cap=131072, ws_bytes=need - 1) == WS
    assert str(need) in err(lib)
    assert dec(lib, cfg_swa(), S=4, cap=128, ws=None, ws_bytes=0) == WS


def test_decode_noalloc_contract(lib):
    """The allocation-free decode validates like mimo_attn_decode and refuses a
    call whose workspace exceeds its 32 MiB scratch, all before any HIP call."""
    def call(cfg, S, cap=131072, q=FAKE):
        return lib.mimo_attn_decode_noalloc(ctypes.byref(cfg), S, q, FAKE, FAKE, FAKE, cap, None, FAKE, None)
    g = cfg_glob()
    assert lib.mimo_attn_decode_workspace_size(ctypes.byref(g), 752, 131072) > 32 << 20
    assert call(g, 752) == WS
    assert "scratch" in err(lib) and str(32 << 20) in err(lib)
    assert call(cfg_swa(), 880, cap=384) == WS
    assert call(g, -1) == INVAL
    assert call(cfg_swa(), 4, cap=64) == INVAL     # ring shorter than the window
    assert call(cfg_swa(num_kv_heads=2), 4, cap=128) == UNSUP
    assert call(g, 4, q=None) == INVAL
    assert call(g, 0, q=None) == OK


def decm(lib, cfg, S=4, nq=4, cap=256, ws=FAKE, ws_bytes=1 << 30, q=FAKE):
    return lib.mimo_attn_decode_multi(ctypes.byref(cfg), S, nq, q, FAKE, FAKE, FAKE, cap, None, FAKE, ws,
                                      ws_bytes, None)


def test_decode_multi_contract(lib):
    assert decm(lib, cfg_swa(), nq=0) == INVAL
    assert decm(lib, cfg_swa(), nq=8, cap=134) == INVAL            # ring shorter than window + n_q - 1
    assert "window + n_q - 1" in err(lib)
    assert decm(lib, cfg_glob(), nq=9) == UNSUP                    # 16 heads x 9 tokens > 128 columns
    assert decm(lib, cfg_swa(), nq=17) == UNSUP                    # 8 heads x 17 tokens
    assert decm(lib, cfg_glob(), S=0, q=None) == OK
    assert decm(lib, cfg_glob(), q=None) == INVAL


def test_decode_multi_workspace(lib):
    def size(cfg, S, nq):
        return lib.mimo_attn_decode_multi_workspace_size(ctypes.byref(cfg), S, nq, 4096)

    def expect(S, nq, groups):
        return (groups + S) * nq * 64 * (128 + 2) * 4 + (S + 1) * 8 + 3 * S * 4 + groups * 4
    # step ranges: 1024 waves over the KV heads and the waves each KV head's columns need
    assert size(cfg_glob(), 16, 1) == lib.mimo_attn_decode_workspace_size(ctypes.byref(cfg_glob()), 16, 4096)
    assert size(cfg_swa(), 64, 8) == expect(64, 8, 1024 // (8 * 2))
    assert size(cfg_glob(), 16, 4) == expect(16, 4, 1024 // (4 * 2))
    assert size(cfg_glob(), 16, 8) == expect(16, 8, 1024 // (4 * 4))
    assert size(cfg_glob(), 16, 9) == 0
    assert decm(lib, cfg_glob(), S=16, nq=4, ws_bytes=expect(16, 4, 128) - 1) == WS


def paged(lib, cfg, S=4, nq=1, block_size=128, dtype=0, ks=1.0, vs=1.0, table=FAKE, max_blocks=8, n_blocks=64,
          ws_bytes=1 << 30):
    return lib.mimo_attn_decode_paged(ctypes.byref(cfg), S, nq, FAKE, FAKE, FAKE, FAKE, n_blocks, block_size,
                                      dtype, ctypes.c_float(ks), ctypes.c_float(vs), table, max_blocks, None, FAKE,
                                      FAKE, ws_bytes, None)


def test_paged_decode_contract(lib):
    assert paged(lib, cfg_glob(), block_size=96) == UNSUP      # not a power of two
    assert paged(lib, cfg_glob(), block_size=16) == UNSUP      # below one 32-slot step
    assert paged(lib, cfg_glob(), dtype=7) == INVAL
    assert paged(lib, cfg_glob(), dtype=1, ks=0.0) == INVAL
    assert paged(lib, cfg_glob(), table=None) == INVAL
    assert paged(lib, cfg_glob(), n_blocks=0) == INVAL
    assert paged(lib, cfg_glob(), max_blocks=1 << 24) == UNSUP   # more than 2^30 slots per sequence
    assert paged(lib, cfg_glob(), ws_bytes=16) == WS
    assert paged(lib, cfg_glob(), S=0, table=None) == OK
    c = cfg_glob()
    assert lib.mimo_kv_paged_append(ctypes.byref(c), 4, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 100, 0,
                                    ctypes.c_float(1.0), ctypes.c_float(1.0), FAKE, 8, None) == UNSUP
    assert lib.mimo_kv_paged_append(ctypes.byref(c), 4, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 128, 0,
                                    ctypes.c_float(1.0), ctypes.c_float(1.0), None, 8, None) == INVAL
    assert lib.mimo_kv_paged_append(ctypes.byref(c), 0, None, None, None, None, None, 64, 128, 1,
                                    ctypes.c_float(1.0), ctypes.c_float(1.0), None, 8, None) == OK


def bwd(lib, cfg, Bn=2, T=64, ws=FAKE, ws_bytes=1 << 30, dsinks=FAKE, sinks=None, lse=FAKE):
    return lib.mimo_attn_prefill_backward(ctypes.byref(cfg), FAKE, FAKE, FAKE, sinks, Bn, T, 0, FAKE, lse, FAKE,
                                          FAKE, FAKE, FAKE, dsinks, ws, ws_bytes, None)


def test_backward_contract(lib):
    c = cfg_swa()
    assert bwd(lib, c, lse=None) == INVAL
    assert bwd(lib, c, sinks=FAKE, dsinks=None) == INVAL
    assert "dsinks" in err(lib)
    assert bwd(lib, c, ws=None, ws_bytes=0) == WS
    need = lib.mimo_attn_backward_workspace_size(ctypes.byref(c), 2, 64)
    rows = 2 * 64 * 64                          # (token, query head) pairs
    # per pair the 64 rotated q dims (bf16) and D; per (token, KV head) the 64 rotated k dims;
    # sink partials per (batch row, 32-token block, head)
    krows = 2 * 64 * c.num_kv_heads
    assert need == (rows + krows) * 64 * 2 + (rows + 2 * 2 * 64) * 4
    for bad in (cfg_swa(num_kv_heads=0), cfg_swa(num_kv_heads=-8), cfg_swa(num_q_heads=60)):
        assert lib.mimo_attn_backward_workspace_size(ctypes.byref(bad), 2, 64) == 0
    assert lib.mimo_attn_backward_workspace_size(ctypes.byref(c), 0, 64) == 0
    assert bwd(lib, c, ws_bytes=need - 1) == WS
    assert bwd(lib, cfg_swa(num_q_heads=16, num_kv_heads=8)) == UNSUP    # group of 2
    assert bwd(lib, c, Bn=1, T=(1 << 24) + 1) == UNSUP                   # B * T * 64 heads past 2^30
    assert bwd(lib, c, Bn=1, T=1 << 24, ws_bytes=0) == WS                # at 2^30 the size is accepted
    assert bwd(lib, c, T=0, lse=None) == OK


def test_rope_and_append_contract(lib):
    c = cfg_swa()
    assert lib.mimo_rope_partial(ctypes.byref(c), FAKE, None, 4, 8, FAKE, None) == INVAL
    assert lib.mimo_rope_partial(ctypes.byref(c), FAKE, FAKE, -1, 8, FAKE, None) == INVAL
    assert lib.mimo_rope_partial(ctypes.byref(c), FAKE, FAKE, 4, 0, FAKE, None) == INVAL
    # partial overlap of input and output
    x = ctypes.c_void_p(0x100000)
    y = ctypes.c_void_p(0x100000 + 384)
    assert lib.mimo_rope_partial(ctypes.byref(c), x, y, 4, 8, FAKE, None) == INVAL
    assert lib.mimo_rope_partial(ctypes.byref(c), FAKE, FAKE, 0, 8, FAKE, None) == OK
    assert lib.mimo_kv_ring_append(ctypes.byref(c), 2, FAKE, FAKE, None, FAKE, FAKE, 128, None) == INVAL
    assert lib.mimo_kv_ring_append(ctypes.byref(c), 2, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == INVAL
    assert lib.mimo_kv_ring_append(ctypes.byref(c), 0, None, None, None, None, None, 128, None) == OK


ODD = ctypes.c_void_p(0x10008)   # 8-byte aligned, not 16


def test_misaligned_pointers_are_rejected(lib):
    """bf16 / fp8 tensors and workspaces move in 16-byte pieces: a pointer that is not
    16-byte aligned is an invalid argument, caught on the host before any launch."""
    calls = {
        "swa q": lambda: swa(lib, cfg_swa(), q=ODD),
        "swa out": lambda: swa(lib, cfg_swa(), out=ODD),
        "global ws": lambda: glob(lib, cfg_glob(), ws=ODD, ws_bytes=1 << 30),
        "varlen q": lambda: varlen(lib, cfg_swa(), q=ODD),
        "decode q": lambda: dec(lib, cfg_glob(), q=ODD),
        "decode ws": lambda: dec(lib, cfg_glob(), ws=ODD),
        "decode_multi q": lambda: decm(lib, cfg_glob(), q=ODD),
        "backward ws": lambda: bwd(lib, cfg_swa(), ws=ODD),
        "rope": lambda: lib.mimo_rope_partial(ctypes.byref(cfg_swa()), ODD, ODD, 4, 8, FAKE, None),
        "ring append": lambda: lib.mimo_kv_ring_append(ctypes.byref(cfg_swa()), 2, ODD, FAKE, FAKE, FAKE, FAKE,
                                                       128, None),
    }
    for name, call in calls.items():
        assert call() == INVAL, name
        assert "16-byte aligned" in err(lib), name
    # empty work is still valid whatever the pointers
    assert swa(lib, cfg_swa(), q=ODD, T=0) == OK


def test_error_message_cleared_on_success(lib):
    assert swa(lib, cfg_swa(), q=None) == INVAL
    assert err(lib) != ""
    assert swa(lib, cfg_swa(), Bn=0) == OK
    assert err(lib) == ""


def test_binding_refuses_missing_library(tmp_path):
    saved = B._lib
    B._lib = None
    try:
        with pytest.raises(ImportError):
            B.load_library(str(tmp_path / "nope.so"))
    finally:
        B._lib = saved
