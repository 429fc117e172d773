"""GPU tests of hga_forward, the one-call forward of a segment (summaries of the
active segment, routing, attention; routing and attention in one work-group per
unit for bf16 with 4 query heads per KV head).

Its outputs must equal, bit for bit, those of the three separate calls
(hga_build_summaries, hga_route, hga_attend_fwd), whose parity against the oracle
the other GPU tests establish: on every small parity case (both head sizes, every
GQA width, both dtypes, empty history, zero and oversized budgets), on histories
of 600 to 2,047 candidate chunks (the two-stage chunk selection), and on the
16K-context layer.  The 16K layer is also checked against the oracle directly.
"""
import numpy as np
import pytest
import torch

import hga_inputs as hi

pytestmark = pytest.mark.gpu

from tests.test_gpu_parity import CASES as PARITY_CASES   # noqa: E402

LONG = {
    # J from 600 to 663 candidate chunks, G = 4: one-wave and two-stage selections
    "bf16_g4_d128_hist38k": dict(seed=91, batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, t_hist=38400,
                                 seg_len=256, top_chunks=16, top_groups=64, chunk_mean_var=0.5),
    # J up to 2,047 (the rollout's last segment), head size 64
    "bf16_g4_d64_hist129k": dict(seed=92, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, t_hist=129024,
                                 seg_len=2048, top_chunks=16, top_groups=64, chunk_mean_var=0.5),
}


@pytest.fixture(scope="module")
def chk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    from tests import hga_check
    import sparse_long_context_hga_amd as hga
    hga.lib()
    return hga_check


def _separate_and_fused(chk, w):
    """The same workload through the three separate calls and through hga_forward."""
    A = chk.DeviceLayer(w)
    A.summaries(0, w.t_hist + w.seg_len)
    A.route()
    A.fwd()
    B = chk.DeviceLayer(w)
    B.summaries(0, w.t_hist)
    B.forward()
    torch.cuda.synchronize()
    return A, B


def _assert_same(A, B, name):
    for field in ("gsum", "csum", "cidx", "gidx", "o", "lse"):
        a, b = getattr(A, field), getattr(B, field)
        assert torch.equal(a, b), f"{name}: {field} of hga_forward differs from the separate calls"


@pytest.mark.parametrize("name", list(PARITY_CASES) + list(LONG))
def test_forward_equals_separate_calls(chk, name):
    kw = PARITY_CASES.get(name) or LONG[name]
    w = hi.random_layer(name=name, backward=False, **kw)
    print(f"case {name}: G={w.group_size} d={w.head_dim} t_hist={w.t_hist} S={w.seg_len}", flush=True)
    A, B = _separate_and_fused(chk, w)
    _assert_same(A, B, name)


def test_forward_qwen3_8b_layer_ctx16k(chk):
    """The 16K layer through hga_forward: bit-identical to the separate calls, and
    against the oracle on every unit (routing accepted; O and LSE on every unit
    whose selection is the oracle's)."""
    w = hi.qwen_16k()
    print(f"workload {w.name}", flush=True)
    A, B = _separate_and_fused(chk, w)
    _assert_same(A, B, w.name)
    gs, cs = chk.oracle_summaries(w)
    T = w.t_hist + w.seg_len
    np.testing.assert_array_equal(chk.to_np(B.gsum)[:, :, :T // 8], gs[:, :, :T // 8])
    np.testing.assert_array_equal(chk.to_np(B.csum)[:, :, :T // 64], cs[:, :, :T // 64])
    cidx, gidx = B.cidx.cpu().numpy(), B.gidx.cpu().numpy()
    ocidx, ogidx, tables = chk.oracle_route(w, gs, cs)
    chk.accept_all_units(w, gs, cs, cidx, gidx, w.name + "_forward", ocidx, tables)
    o_fused, lse_fused = chk.to_np(B.o), chk.to_np(B.lse)
    A.fwd(torch.from_numpy(ogidx).cuda())
    torch.cuda.synchronize()
    o, lse = chk.to_np(A.o), chk.to_np(A.lse)
    n_same = chk.chain_matches(w, gidx, ogidx, o_fused, lse_fused, o, lse)
    eo, el = chk.fwd_errors(w, o, lse, ogidx)
    print(f"O max-abs {eo:.3e} LSE max-abs {el:.3e}; fused forward bit-identical on {n_same} units", flush=True)
    assert eo <= chk.TOL_O["bf16"] and el <= chk.TOL_O["bf16"]
    assert n_same >= w.batch * w.n_kv_heads * w.seg_len // 64 - 2


def test_forward_timed_events(chk):
    """hga_forward with its four dispatch events: same outputs, ordered timestamps."""
    import sparse_long_context_hga_amd as hga
    w = hi.random_layer(name="timed", backward=False, **PARITY_CASES["bf16_g4_d128_ragged"])
    A, B = _separate_and_fused(chk, w)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(hga.HGA_FWD_EVENTS)]
    B.forward(events=ev)
    torch.cuda.synchronize()
    _assert_same(A, B, "timed")
    t = [ev[0].elapsed_time(e) for e in ev]
    assert 0.0 <= t[1] <= t[2] <= t[3], t
