"""Host-side argument checks of the Python binding and the layer plumbing (no GPU
needed): a tensor whose dtype, layout, size or device does not match the call is
rejected with a Python error before any pointer reaches the library, because the
library trusts pointers and would otherwise read or write out of bounds."""
import pytest
import torch

import sparse_long_context_hga_amd as hga
from sparse_long_context_hga_amd import _lib
from sparse_long_context_hga_amd.layer import HGADecoder, HGAKVCache, hga_attention


def test_make_shape_accepts_only_known_dtypes():
    assert hga.make_shape(1, 4, 1, 64, 2, 8, "bf16").dtype == hga.HGA_BF16
    assert hga.make_shape(1, 4, 1, 64, 2, 8, "f32").dtype == hga.HGA_F32
    for bad in ("bfloat16", "fp16", "float32", "BF16", ""):
        with pytest.raises(ValueError):
            hga.make_shape(1, 4, 1, 64, 2, 8, bad)


def test_tensor_check_rejects_dtype_layout_and_size():
    t = torch.zeros(4, 8, dtype=torch.bfloat16)
    _lib._need("f", "t", t, torch.bfloat16, 32, None)                  # passes
    with pytest.raises(ValueError, match="dtype"):
        _lib._need("f", "t", t, torch.float32, 32, None)
    with pytest.raises(ValueError, match="contiguous"):
        _lib._need("f", "t", t.t(), torch.bfloat16, 32, None)
    with pytest.raises(ValueError, match="elements"):
        _lib._need("f", "t", t, torch.bfloat16, 33, None)
    with pytest.raises(ValueError, match="required"):
        _lib._need("f", "t", None, torch.bfloat16, 32, None)
    _lib._need("f", "t", None, torch.bfloat16, 32, None, optional=True)
    with pytest.raises(ValueError, match="on"):
        _lib._need("f", "t", t, torch.bfloat16, 32, torch.device("cuda", 0))


def test_wrappers_reject_host_tensors_before_the_library():
    s = hga.make_shape(1, 4, 1, 64, 2, 8, "bf16")
    k = torch.zeros(1, 1, 256, 64, dtype=torch.bfloat16)
    gs = torch.zeros(1, 1, 32, 64, dtype=torch.bfloat16)
    cs = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="ROCm device"):
        hga.hga_build_summaries(s, k, 256, 0, 256, gs, cs)
    q = torch.zeros(1, 4, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="ROCm device"):
        hga.hga_route(s, q, cs, gs, 256, 128, 128, None, None)
    cidx = torch.zeros(1, 1, 2, 2, dtype=torch.int32)
    gidx = torch.zeros(1, 1, 2, 8, dtype=torch.int32)
    o = torch.zeros_like(q)
    lse = torch.zeros(1, 4, 128, dtype=torch.float32)
    with pytest.raises(ValueError, match="ROCm device"):
        hga.hga_forward_causal(s, q, None, k, k, cs, gs, 256, 128, 128, cidx, gidx, o, lse)


def test_layer_op_rejects_mismatches_before_any_launch():
    cache = HGAKVCache(1, 2, 64, 256, torch.bfloat16, device="cpu")
    q = torch.zeros(1, 4, 128, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        hga_attention(q.float(), k, k, cache, 1, 8)                      # fp32 q on a bf16 cache
    with pytest.raises(ValueError, match="does not match"):
        hga_attention(torch.zeros(1, 4, 128, 128, dtype=torch.bfloat16), k, k, cache, 1, 8)
    with pytest.raises(ValueError, match="k_seg"):
        hga_attention(q, torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16), k, cache, 1, 8)
    with pytest.raises(ValueError, match="v_seg"):
        hga_attention(q, k, k.float(), cache, 1, 8)
    with pytest.raises(ValueError, match="multiple of 64"):
        hga_attention(q[:, :, :100], k, k, cache, 1, 8)
    with pytest.raises(ValueError, match="KV heads"):
        hga_attention(torch.zeros(1, 3, 128, 64, dtype=torch.bfloat16), k, k, cache, 1, 8)
    assert cache.length == 0


def test_decoder_step_rejects_mismatches():
    cache = HGAKVCache(2, 1, 64, 256, torch.bfloat16, device="cpu")
    dec = HGADecoder(cache, n_q_heads=4, top_chunks=2, top_groups=8)
    kv = torch.zeros(2, 1, 64, dtype=torch.bfloat16)
    pos = torch.tensor([5, 9], dtype=torch.int32)
    with pytest.raises(ValueError, match="q must be"):
        dec.step(torch.zeros(2, 4, 64, dtype=torch.float32), kv, kv, pos)   # fp32 q on a bf16 cache
    with pytest.raises(ValueError, match="k_new"):
        dec.step(torch.zeros(2, 4, 64, dtype=torch.bfloat16), kv[:1], kv, pos)
    with pytest.raises(ValueError, match="pos"):
        dec.step(torch.zeros(2, 4, 64, dtype=torch.bfloat16), kv, kv, pos.long())


def test_stack_checks_budgets():
    from sparse_long_context_hga_amd.layer import HGAStack
    layers = [object(), object()]
    with pytest.raises(ValueError, match="budgets"):
        HGAStack(layers, batch=1, n_kv_heads=1, head_dim=64, t_cap=256, budgets=[(2, 8)], device="cpu")
    st = HGAStack(layers, batch=1, n_kv_heads=1, head_dim=64, t_cap=256, budgets=(2, 8), device="cpu")
    assert st.budgets == [(2, 8), (2, 8)] and st.length == 0 and len(st.caches) == 2
