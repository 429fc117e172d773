"""GPU parity on small layers whose shapes Hypothesis draws (derandomized, so every
run checks the same examples): 1-2 sequences, 1-2 KV heads, 1, 2, 4 or 8 query heads
per KV head, head size 64 or 128, bf16 or fp32, up to 1,024 history and 512 active
tokens (multiples of 64), chunk budgets 0-6 and group budgets 0-8 k_c, plain or
block-structured keys.  Each example checks every step against the oracle:

- summaries of the history and the active segment bit for bit;
- routing on the oracle's summaries, accepted with the near-tie rule;
- the forward and the backward on the oracle's selection, to the parity tolerances
  (per query block and per active chunk for the gradients);
- hga_forward and hga_forward_causal bit for bit against the separate calls.

HGA_HYPOTHESIS_EXAMPLES sets the number of examples (default 100; 600 have been run).
"""
import os

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import hga_inputs as hi

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def chk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    from tests import hga_check
    import sparse_long_context_hga_amd as hga
    hga.lib()
    return hga_check


@st.composite
def small_layers(draw):
    G = draw(st.sampled_from([1, 2, 4, 8]))
    hkv = draw(st.integers(1, 2))
    kc = draw(st.integers(0, 6))
    return dict(seed=draw(st.integers(0, 2 ** 16)), batch=draw(st.integers(1, 2)), n_q_heads=G * hkv,
                n_kv_heads=hkv, head_dim=draw(st.sampled_from([64, 128])),
                t_hist=64 * draw(st.integers(0, 16)), seg_len=64 * draw(st.integers(1, 8)),
                top_chunks=kc, top_groups=draw(st.integers(0, 8 * kc)),
                dtype=draw(st.sampled_from(["bf16", "f32"])),
                chunk_mean_var=draw(st.sampled_from([0.0, 0.5])))


@settings(max_examples=int(os.environ.get("HGA_HYPOTHESIS_EXAMPLES", 100)), deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(kw=small_layers())
def test_random_small_layer(chk, kw):
    w = hi.random_layer(name="hypothesis", **kw)
    print(f"case {kw}", flush=True)
    T = w.t_hist + w.seg_len

    # summaries, bit for bit
    gs, cs = chk.oracle_summaries(w)
    L = chk.DeviceLayer(w)
    L.summaries(0, w.t_hist)
    L.summaries(w.t_hist, T)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(chk.to_np(L.gsum)[:, :, :T // 8], gs[:, :, :T // 8])
    np.testing.assert_array_equal(chk.to_np(L.csum)[:, :, :T // 64], cs[:, :, :T // 64])

    # routing on the oracle's summaries, with the near-tie acceptance rule
    L.route(chk.to_dev(cs, w.dtype), chk.to_dev(gs, w.dtype))
    torch.cuda.synchronize()
    cidx, gidx = L.cidx.cpu().numpy(), L.gidx.cpu().numpy()
    for b in range(w.batch):
        for kvh in range(w.n_kv_heads):
            for j in range(w.seg_len // 64):
                chk.check_route_unit(w, gs, cs, b, kvh, j, cidx[b, kvh, j], gidx[b, kvh, j])

    # forward and backward on the oracle's selection
    _, ogidx, _ = chk.oracle_route(w, gs, cs)
    g = torch.from_numpy(ogidx).cuda()
    L.fwd(g)
    L.bwd(g)
    torch.cuda.synchronize()
    eo, el = chk.fwd_errors(w, chk.to_np(L.o), chk.to_np(L.lse), ogidx)
    assert eo <= chk.TOL_O[w.dtype] and el <= chk.TOL_O[w.dtype], (eo, el)
    errs = chk.bwd_errors(w, chk.to_np(L.dq), chk.to_np(L.dk), chk.to_np(L.dv), ogidx)
    chk.assert_grads(errs, chk.TOL_GRAD_REL_L2 if w.dtype == "bf16" else 1e-4)

    # hga_forward against the separate calls
    A = chk.DeviceLayer(w)
    A.summaries(0, T)
    A.route()
    A.fwd()
    B = chk.DeviceLayer(w)
    B.summaries(0, w.t_hist)
    B.forward()
    torch.cuda.synchronize()
    for field in ("gsum", "csum", "cidx", "gidx", "o", "lse"):
        assert torch.equal(getattr(A, field), getattr(B, field)), f"hga_forward: {field} differs"

    # hga_forward_causal against summaries + hga_route_causal + hga_attend_fwd
    qp = None
    if w.t_hist > 0:
        qp = chk.to_dev(hi.prev_query_block(seed=kw["seed"] + 1, batch=w.batch, n_q_heads=w.n_q_heads,
                                            head_dim=w.head_dim, dtype=w.dtype), w.dtype)
    A = chk.DeviceLayer(w)
    A.summaries(0, T)
    A.route_causal(qp)
    A.fwd()
    B = chk.DeviceLayer(w)
    B.summaries(0, w.t_hist)
    B.forward_causal(qp)
    torch.cuda.synchronize()
    for field in ("gsum", "csum", "cidx", "gidx", "o", "lse"):
        assert torch.equal(getattr(A, field), getattr(B, field)), f"hga_forward_causal: {field} differs"
