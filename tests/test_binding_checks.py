"""The Python binding checks every tensor before it hands a pointer to the
library (which takes plain pointers and sizes and cannot see a tensor that is
too small).  Host tensors are enough to show it: a wrongly sized tensor raises
ValueError, and a call whose shapes are all right stops at the first device
check (TypeError: not a GPU tensor), so no call here reaches a launch.
"""
import pytest
import torch

import hybrid_linear_attention_lightning_amd as la

B, H, N, d = 1, 2, 64, 64


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def f32(*shape):
    return t(*shape, dtype=torch.float32)


def qkv(*shape):
    return t(*shape), t(*shape), t(*shape)


def test_prefill_shapes():
    q, k, v = qkv(B, H, N, d)
    s = f32(H)
    with pytest.raises(ValueError):
        la.prefill(q, t(B, H, N + 1, d), v, s)
    with pytest.raises(ValueError):
        la.prefill(q, k, v, f32(H + 1))
    with pytest.raises(ValueError):
        la.prefill(q, k, v, s, state_in=f32(B, H, d, d - 1))
    with pytest.raises(ValueError):
        la.prefill(q, k, v, s, out=t(B, H, N - 1, d))
    with pytest.raises(ValueError):
        la.prefill(q, k, v, s, state_out=f32(B + 1, H, d, d))
    with pytest.raises(TypeError):
        la.prefill(q, k, v, s, state_in=t(B, H, d, d))  # state must be fp32
    with pytest.raises(ValueError):
        la.prefill(t(B, H, N), k, v, s)  # q must be 4-d
    with pytest.raises(TypeError, match="GPU"):
        la.prefill(q, k, v, s, state_in=f32(B, H, d, d))


def test_prefill_gated_shapes():
    q, k, v = qkv(B, H, N, d)
    s, g, w = f32(H), t(B, H, N, d), f32(H, d)
    with pytest.raises(ValueError):
        la.prefill_gated(q, k, v, s, t(B, H, N, d - 1), w)
    with pytest.raises(ValueError):
        la.prefill_gated(q, k, v, s, g, f32(H, d + 1))
    with pytest.raises(TypeError, match="GPU"):
        la.prefill_gated(q, k, v, s, g, w)


def test_prefill_halves_shapes():
    q, k, v = qkv(B, H, N, d)
    s = f32(H)
    with pytest.raises(ValueError):
        la.prefill_prepass(k, t(B, H, N, d + 1), s, 64, None)
    with pytest.raises(ValueError):
        la.prefill_main(q, k, v, s, 64, None, t(B, H, N, 2 * d))
    with pytest.raises(TypeError, match="GPU"):
        la.prefill_main(q, k, v, s, 64, None, t(B, H, N, d))


def test_decode_shapes():
    q, k, v = qkv(B, H, d)
    s, st = f32(H), f32(B, H, d, d)
    with pytest.raises(ValueError):
        la.decode_step(q, k, v, s, f32(B, H, d, d // 2))
    with pytest.raises(ValueError):
        la.decode_step(q, k, v, s, st, out=t(B, H + 1, d))
    with pytest.raises(ValueError):
        la.decode_step(q, k, v, f32(2 * H), st)
    with pytest.raises(ValueError):
        la.decode_step(q, t(B, H, d - 8), v, s, st)
    with pytest.raises(TypeError, match="GPU"):
        la.decode_step(q, k, v, s, st)


def test_decode_tokens_shapes():
    q, k, v = qkv(B, H, 4, d)
    s, st = f32(H), f32(B, H, d, d)
    with pytest.raises(ValueError):
        la.decode_tokens(q, k, v, s, f32(B, H, d + 1, d))
    with pytest.raises(ValueError):
        la.decode_tokens(q, k, v, s, st, out=t(B, H, 3, d))
    with pytest.raises(TypeError, match="GPU"):
        la.decode_tokens(q, k, v, s, st)


def test_backward_shapes():
    q, k, v = qkv(B, H, N, d)
    g, s = t(B, H, N, d), f32(H)
    with pytest.raises(ValueError):
        la.prefill_bwd(q, k, v, t(B, H, N, d // 2), s)
    with pytest.raises(ValueError):
        la.prefill_bwd(q, k, v, g, s, dq=t(B, H, N - 1, d))
    with pytest.raises(ValueError):
        la.prefill_bwd(q, k, v, g, s, dv=t(B, 2 * H, N, d))
    with pytest.raises(TypeError, match="GPU"):
        la.prefill_bwd(q, k, v, g, s)


def test_varlen_token_count_and_states():
    T = 300
    q, k, v = qkv(H, T, d)
    s = f32(H)
    with pytest.raises(ValueError, match="cu_seqlens"):
        la.prefill_varlen(q, k, v, s, [0, 100, T + 1])  # would address past the tensors
    with pytest.raises(ValueError, match="cu_seqlens"):
        la.prefill_varlen(q, k, v, s, [0, 100, T - 1])
    with pytest.raises(ValueError):
        la.prefill_varlen(q, k, v, s, [0])
    with pytest.raises(ValueError):
        la.prefill_varlen(q, k, v, s, [0, 100, T], state_in=f32(3, H, d, d))  # 2 sequences
    with pytest.raises(ValueError):
        la.prefill_varlen(q, k, v, s, [0, 100, T], state_out=f32(2, H, d, d + 1))
    with pytest.raises(TypeError, match="GPU"):
        la.prefill_varlen(q, k, v, s, [0, 100, T])
    g = t(H, T, d)
    with pytest.raises(ValueError, match="cu_seqlens"):
        la.prefill_bwd_varlen(q, k, v, g, s, [0, T + 64])
    with pytest.raises(ValueError):
        la.prefill_bwd_varlen(q, k, v, g, s, [0, T], dk=t(H, T + 1, d))
    with pytest.raises(TypeError, match="GPU"):
        la.prefill_bwd_varlen(q, k, v, g, s, [0, T])


def test_workspace_is_never_replaced():
    dev = torch.device("cpu")
    with pytest.raises(ValueError, match="needed"):
        la._workspace(1000, dev, torch.empty(999, dtype=torch.uint8))
    with pytest.raises(ValueError, match="earlier call"):
        la._workspace(1000, dev, None, required=True)
    # a caller's workspace that is large enough is used as it is
    with pytest.raises(ValueError, match="GPU"):
        la._workspace(1000, torch.device("cuda:0"), torch.empty(1000, dtype=torch.uint8))
    assert la._workspace(0, dev, None, required=True) == (None, 0)
