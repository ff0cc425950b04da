"""Argument checks of the Python binding that run before anything reaches the device: ranks,
shapes and dtypes raise, and host tensors are refused (the binding passes device pointers
only, and there is no host fallback)."""
import pytest
import torch

import paged_kv_cache_127_amd as pkv


def _args(S=2, Hq=8, Hkv=2, d=64, B=16, N=8, dt=torch.bfloat16):
    q = torch.zeros(S, Hq, d, dtype=dt)
    out = torch.zeros(S, Hq, d, dtype=torch.float32)
    kp = torch.zeros(N, Hkv, B, d, dtype=dt)
    vp = torch.zeros(N, Hkv, B, d, dtype=dt)
    tab = torch.zeros(S, 4, dtype=torch.int32)
    lens = torch.ones(S, dtype=torch.int32)
    ws = torch.zeros(256, dtype=torch.uint8)
    return out, q, kp, vp, tab, lens, ws


def test_decode_shape_and_dtype_errors():
    out, q, kp, vp, tab, lens, ws = _args()
    with pytest.raises(ValueError):                       # q of the wrong rank
        pkv.paged_attn_decode(out, q[0], kp, vp, tab, lens, 16, workspace=ws)
    with pytest.raises(ValueError):                       # pools of different shapes
        pkv.paged_attn_decode(out, q, kp, vp[:, :1], tab, lens, 16, workspace=ws)
    with pytest.raises(ValueError):                       # head dims of q and the pools differ
        pkv.paged_attn_decode(out, q[..., :32].contiguous(), kp, vp, tab, lens, 16,
                              workspace=ws)
    with pytest.raises(ValueError):                       # one table row short
        pkv.paged_attn_decode(out, q, kp, vp, tab[:1], lens, 16, workspace=ws)
    with pytest.raises(TypeError):                        # output neither fp32 nor the cache type
        pkv.paged_attn_decode(out.half(), q, kp, vp, tab, lens, 16, workspace=ws)
    with pytest.raises(TypeError):                        # no such cache element type
        pkv.paged_attn_decode(out, q, kp.to(torch.int8), vp.to(torch.int8), tab, lens, 16,
                              workspace=ws)


def test_host_tensors_are_refused():
    out, q, kp, vp, tab, lens, ws = _args()
    with pytest.raises(ValueError, match="device tensor"):
        pkv.paged_attn_decode(out, q, kp, vp, tab, lens, 16, workspace=ws)
