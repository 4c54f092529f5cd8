"""The Python binding refuses tensors whose shapes disagree with the call's sizes and the
layer configuration, and a workspace in host memory, before anything reaches the library:
a kernel takes its sizes from the C arguments and would index past a tensor made too small.
No kernel is launched by these tests."""
import pytest
import torch

from global_attention_sinks_amd import binding as Bd

pytestmark = pytest.mark.gpu


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device="cuda")


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32, device="cuda")


def i64(*shape):
    return torch.zeros(shape, dtype=torch.int64, device="cuda")


def test_prefill_shapes_are_checked():
    c = Bd.swa_cfg()
    q, k, v, out = bf16(1, 64, 64, 192), bf16(1, 64, 8, 192), bf16(1, 64, 8, 128), bf16(1, 64, 64, 128)
    with pytest.raises(ValueError, match="k must have shape"):
        Bd.mimo_attn_prefill_swa(c, q, bf16(1, 63, 8, 192), v, None, out)
    with pytest.raises(ValueError, match="v must have shape"):
        Bd.mimo_attn_prefill_swa(c, q, k, bf16(1, 64, 4, 128), None, out)
    with pytest.raises(ValueError, match="sinks must have shape"):
        Bd.mimo_attn_prefill_swa(c, q, k, v, f32(32), out)
    with pytest.raises(ValueError, match="lse must have shape"):
        Bd.mimo_attn_prefill_swa(c, q, k, v, None, out, lse=f32(1, 64, 63))
    g = Bd.global_cfg()
    with pytest.raises(ValueError, match="q must have shape"):       # 8 KV heads against a 4-head layer
        Bd.mimo_attn_prefill_global(g, bf16(1, 64, 32, 192), bf16(1, 64, 4, 192), bf16(1, 64, 4, 128), out)
    with pytest.raises(ValueError, match="ws must be a contiguous CUDA tensor"):
        Bd.mimo_attn_prefill_global(g, q, bf16(1, 64, 4, 192), bf16(1, 64, 4, 128), out,
                                    ws=torch.zeros(1 << 20, dtype=torch.uint8))


def test_backward_shapes_are_checked():
    c = Bd.swa_cfg()
    q, k, v, o = bf16(1, 32, 64, 192), bf16(1, 32, 8, 192), bf16(1, 32, 8, 128), bf16(1, 32, 64, 128)
    lse = f32(1, 64, 32)
    with pytest.raises(ValueError, match="dk must have shape"):
        Bd.mimo_attn_prefill_backward(c, q, k, v, None, o, lse, o, bf16(1, 32, 64, 192), bf16(1, 32, 8, 128),
                                      bf16(1, 32, 8, 128))
    with pytest.raises(ValueError, match="dsinks must have shape"):
        Bd.mimo_attn_prefill_backward(c, q, k, v, f32(64), o, lse, o, bf16(1, 32, 64, 192), bf16(1, 32, 8, 192),
                                      bf16(1, 32, 8, 128), f32(8))


def test_decode_and_append_shapes_are_checked():
    c = Bd.swa_cfg()
    S, cap = 4, 128
    q, out, pos = bf16(S, 64, 192), bf16(S, 64, 128), i64(S)
    kc, vc = bf16(S, cap, 8, 192), bf16(S, cap, 8, 128)
    ws = torch.zeros(Bd.mimo_attn_decode_workspace_size(c, S, cap), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="k_cache must have shape"):
        Bd.mimo_attn_decode(c, q, pos, bf16(S - 1, cap, 8, 192), vc, None, out, ws=ws)
    with pytest.raises(ValueError, match="v_cache must have shape"):
        Bd.mimo_attn_decode_noalloc(c, q, pos, kc, bf16(S, cap - 1, 8, 128), None, out)
    with pytest.raises(ValueError, match="q_pos must have shape"):
        Bd.mimo_attn_decode_multi(c, bf16(S, 2, 64, 192), i64(S + 1), kc, vc, None, bf16(S, 2, 64, 128), ws=ws)
    with pytest.raises(ValueError, match="ws must be a contiguous CUDA tensor"):
        Bd.mimo_attn_decode(c, q, pos, kc, vc, None, out, ws=ws.cpu())
    with pytest.raises(ValueError, match="v_new must have shape"):
        Bd.mimo_kv_ring_append(c, bf16(S, 8, 192), bf16(S, 8, 192), pos, kc, vc)
    kp, vp = bf16(16, 32, 8, 192), bf16(16, 32, 8, 128)
    table = torch.zeros((S, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="block_table must have shape"):
        Bd.mimo_kv_paged_append(c, bf16(S, 8, 192), bf16(S, 8, 128), pos, kp, vp, table[:2])
    with pytest.raises(ValueError, match="v_pool must have shape"):
        Bd.mimo_attn_decode_paged(c, bf16(S, 1, 64, 192), pos, kp, bf16(16, 64, 8, 128), table, None,
                                  bf16(S, 1, 64, 128), ws=ws)
