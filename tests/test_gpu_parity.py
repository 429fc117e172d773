"""GPU parity of every step of the hot path against the CPU oracle, on seeded
layers small enough for the oracle to finish in seconds yet spanning several
tiles and ragged tails (history not a multiple of the 32-chunk score tile, group
budgets not a multiple of the 8-group key tile, blocks with fewer candidates than
the budget, an empty history, a zero budget, every GQA width and head size).

Expected values come only from the oracle.  Attention and gradients are checked
on the oracle's own selection (passed to the library as its group_idx input), so
a legitimate near-tie difference in routing cannot cascade; routing is checked
separately with the near-tie acceptance rule.
"""
import numpy as np
import pytest
import torch

import hga_inputs as hi
from oracle import hga_oracle as ora

pytestmark = pytest.mark.gpu

CASES = {
    # name: random_layer kwargs
    "bf16_g4_d128_ragged": dict(seed=1, batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, t_hist=1088,
                                seg_len=384, top_chunks=5, top_groups=27, chunk_mean_var=0.5),
    "bf16_g2_d128_b2_multitile": dict(seed=2, batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128,
                                      t_hist=2112, seg_len=512, top_chunks=16, top_groups=64),
    "bf16_g1_d64_b2": dict(seed=3, batch=2, n_q_heads=2, n_kv_heads=2, head_dim=64, t_hist=640,
                           seg_len=256, top_chunks=3, top_groups=13),
    "bf16_g8_d128": dict(seed=4, batch=1, n_q_heads=8, n_kv_heads=1, head_dim=128, t_hist=256,
                         seg_len=256, top_chunks=2, top_groups=9),
    "bf16_g4_d64": dict(seed=5, batch=1, n_q_heads=8, n_kv_heads=2, head_dim=64, t_hist=512,
                        seg_len=192, top_chunks=6, top_groups=41, chunk_mean_var=0.5),
    "bf16_hist0": dict(seed=6, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128, t_hist=0,
                       seg_len=512, top_chunks=4, top_groups=20),
    "bf16_zero_budget": dict(seed=7, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128, t_hist=256,
                             seg_len=192, top_chunks=0, top_groups=0),
    "bf16_budget_exceeds_candidates": dict(seed=8, batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128,
                                           t_hist=128, seg_len=256, top_chunks=64, top_groups=512),
    "bf16_single_block": dict(seed=9, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128, t_hist=1024,
                              seg_len=64, top_chunks=7, top_groups=50, t_cap=2048),
    # every block selects every earlier chunk and group: the segment's first chunks are
    # attended by up to 16 blocks x 8 heads = 128 rounds, cut into the maximum of 8
    # dK/dV items each (items of 16 rounds, partial sums of 8 parts)
    "bf16_g8_full_coverage": dict(seed=13, batch=1, n_q_heads=8, n_kv_heads=1, head_dim=128, t_hist=0,
                                  seg_len=1024, top_chunks=16, top_groups=128),
    "f32_g1_d64": dict(seed=10, batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64, t_hist=320,
                       seg_len=256, top_chunks=3, top_groups=19, dtype="f32"),
    "f32_g4_d128": dict(seed=11, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128, t_hist=256,
                        seg_len=128, top_chunks=3, top_groups=17, dtype="f32"),
    "f32_g2_d64_hist0": dict(seed=12, batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, t_hist=0,
                             seg_len=320, top_chunks=2, top_groups=11, dtype="f32"),
}


@pytest.fixture(scope="module")
def chk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    from tests import hga_check
    import sparse_long_context_hga_amd as hga
    hga.lib()
    return hga_check


@pytest.fixture(scope="module")
def cases(chk):
    out = {}
    for name, kw in CASES.items():
        w = hi.random_layer(name=name, **kw)
        gs, cs = chk.oracle_summaries(w)
        cidx, gidx, _ = chk.oracle_route(w, gs, cs)
        out[name] = (w, gs, cs, cidx, gidx)
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_summaries_bit_exact(chk, cases, name):
    w, gs, cs, _, _ = cases[name]
    print(f"case {name}", flush=True)
    L = chk.DeviceLayer(w)
    T = w.t_hist + w.seg_len
    L.summaries(0, w.t_hist)          # history once
    L.summaries(w.t_hist, T)          # then the active segment
    torch.cuda.synchronize()
    np.testing.assert_array_equal(chk.to_np(L.gsum)[:, :, :T // 8], gs[:, :, :T // 8])
    np.testing.assert_array_equal(chk.to_np(L.csum)[:, :, :T // 64], cs[:, :, :T // 64])
    assert not chk.to_np(L.gsum)[:, :, T // 8:].any()            # rows beyond the range untouched


@pytest.mark.parametrize("name", list(CASES))
def test_route_accepted(chk, cases, name):
    w, gs, cs, _, _ = cases[name]
    print(f"case {name}", flush=True)
    L = chk.DeviceLayer(w)
    gs_d = chk.to_dev(gs, w.dtype)
    cs_d = chk.to_dev(cs, w.dtype)
    L.route(cs_d, gs_d)
    torch.cuda.synchronize()
    cidx = L.cidx.cpu().numpy()
    gidx = L.gidx.cpu().numpy()
    cscore = L.cscore.cpu().numpy()
    exempt = 0
    for b in range(w.batch):
        for kvh in range(w.n_kv_heads):
            for j in range(w.seg_len // 64):
                exempt += chk.check_route_unit(w, gs, cs, b, kvh, j, cidx[b, kvh, j], gidx[b, kvh, j])
                # reported scores of the selected chunks match the oracle's fp32 scores
                J = w.t_hist // 64 + j
                sig = ora.block_scores(ora.block_rows(w.q, b, kvh, j, w.group_size), cs[b, kvh, :J])
                for i, c in enumerate(cidx[b, kvh, j]):
                    if c >= 0:
                        assert abs(cscore[b, kvh, j, i] - sig[c]) <= 1e-5 * max(1.0, abs(sig[c]))
                    else:
                        assert cscore[b, kvh, j, i] == -np.inf
    print(f"near-tie exemptions: {exempt}")


LONG_HISTORY = {
    # the blocks' candidate counts J span each regime of the chunk selection: the
    # two-stage selection at 4, 8, 16 and 32 candidates per lane, the last at the
    # library's maximum of 8,192 chunks
    "j600_kc64": dict(t_hist=600 * 64, top_chunks=64, top_groups=100),
    "j1500_kc16": dict(t_hist=1500 * 64, top_chunks=16, top_groups=64),
    "j3000_kc33": dict(t_hist=3000 * 64, top_chunks=33, top_groups=200),
    "j8188_kc64": dict(t_hist=8188 * 64, top_chunks=64, top_groups=511),
}


@pytest.mark.parametrize("name", list(LONG_HISTORY))
def test_route_long_history(chk, name):
    """Routing over histories of 600 to 8,191 candidate chunks: every unit accepted
    against the oracle's scores, and the reported chunk scores match them."""
    w = hi.random_layer(seed=70, batch=1, n_q_heads=2, n_kv_heads=1, head_dim=64, seg_len=256,
                        chunk_mean_var=0.5, backward=False, name=name, **LONG_HISTORY[name])
    print(f"case {name}", flush=True)
    gs, cs = chk.oracle_summaries(w)
    L = chk.DeviceLayer(w)
    L.summaries(0, w.t_hist + w.seg_len)
    L.route()
    torch.cuda.synchronize()
    cidx, gidx, cscore = L.cidx.cpu().numpy(), L.gidx.cpu().numpy(), L.cscore.cpu().numpy()
    exempt = 0
    for j in range(w.seg_len // 64):
        exempt += chk.check_route_unit(w, gs, cs, 0, 0, j, cidx[0, 0, j], gidx[0, 0, j])
        J = w.t_hist // 64 + j
        sig = ora.block_scores(ora.block_rows(w.q, 0, 0, j, w.group_size), cs[0, 0, :J])
        assert np.all(cidx[0, 0, j] >= 0)
        for i, c in enumerate(cidx[0, 0, j]):
            assert abs(cscore[0, 0, j, i] - sig[c]) <= 1e-5 * max(1.0, abs(sig[c]))
    print(f"near-tie exemptions: {exempt}")


@pytest.mark.parametrize("name", list(CASES))
def test_forward_on_oracle_selection(chk, cases, name):
    w, _, _, _, gidx = cases[name]
    print(f"case {name}", flush=True)
    L = chk.DeviceLayer(w)
    L.fwd(torch.from_numpy(gidx).cuda())
    torch.cuda.synchronize()
    eo, el = chk.fwd_errors(w, chk.to_np(L.o), chk.to_np(L.lse), gidx)
    print(f"O max-abs {eo:.3e} LSE max-abs {el:.3e}")
    assert eo <= chk.TOL_O[w.dtype] and el <= chk.TOL_O[w.dtype]


@pytest.mark.parametrize("name", list(CASES))
def test_backward_on_oracle_selection(chk, cases, name):
    w, _, _, _, gidx = cases[name]
    print(f"case {name}", flush=True)
    L = chk.DeviceLayer(w)
    g = torch.from_numpy(gidx).cuda()
    L.fwd(g)
    L.bwd(g)
    torch.cuda.synchronize()
    errs = chk.bwd_errors(w, chk.to_np(L.dq), chk.to_np(L.dk), chk.to_np(L.dv), gidx)
    print(f"grad rel-L2 {errs}")
    tol = chk.TOL_GRAD_REL_L2 if w.dtype == "bf16" else 1e-4
    chk.assert_grads(errs, tol)


@pytest.mark.parametrize("name", ["bf16_g4_d128_ragged", "bf16_g2_d128_b2_multitile", "f32_g1_d64"])
def test_full_chain_and_determinism(chk, cases, name):
    """GPU summaries -> GPU route -> GPU attention; compared with the oracle chain
    wherever the two selections agree exactly, and bitwise repeatable."""
    w, gs, cs, ocidx, ogidx = cases[name]
    print(f"case {name}", flush=True)
    L = chk.DeviceLayer(w)
    L.summaries(0, w.t_hist + w.seg_len)
    L.route()
    L.fwd()
    L.bwd()
    torch.cuda.synchronize()
    first = [chk.to_np(t).copy() for t in (L.gidx, L.o, L.lse, L.dq, L.dk, L.dv)]
    gidx = L.gidx.cpu().numpy()
    same = np.all(gidx == ogidx, axis=-1)
    assert same.mean() > 0.95, f"only {same.mean():.2%} of units selected identically"
    o, lse = ora.attend_fwd(w.q, w.k_cache, w.v_cache, w.t_hist, ogidx, w.softmax_scale, w.group_size)
    G = w.group_size
    og, lg = chk.to_np(L.o), chk.to_np(L.lse)
    for b in range(w.batch):
        for kvh in range(w.n_kv_heads):
            for j in range(w.seg_len // 64):
                if same[b, kvh, j]:
                    sl = (b, slice(kvh * G, kvh * G + G), slice(64 * j, 64 * j + 64))
                    assert np.max(np.abs(og[sl] - o[sl])) <= chk.TOL_O[w.dtype]
                    assert np.max(np.abs(lg[sl] - lse[sl])) <= chk.TOL_O[w.dtype]
    for _ in range(2):
        L.step()
        torch.cuda.synchronize()
        again = [chk.to_np(t) for t in (L.gidx, L.o, L.lse, L.dq, L.dk, L.dv)]
        for a, b_ in zip(first, again):
            assert np.array_equal(a, b_)


@pytest.mark.parametrize("name", ["bf16_g4_d128_ragged", "f32_g4_d128"])
def test_timed_backward_matches(chk, cases, name):
    """hga_attend_bwd_timed writes the same bits as hga_attend_bwd and records its
    events in launch order (dQ, dK/dV, partial sums)."""
    import sparse_long_context_hga_amd as hga
    w, _, _, _, gidx = cases[name]
    print(f"case {name}", flush=True)
    L = chk.DeviceLayer(w)
    g = torch.from_numpy(gidx).cuda()
    L.fwd(g)
    L.bwd(g)
    torch.cuda.synchronize()
    ref = [chk.to_np(t).copy() for t in (L.dq, L.dk, L.dv)]
    for t in (L.dq, L.dk, L.dv):
        t.zero_()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * hga.HGA_BWD_KERNELS)]
    start = torch.cuda.Event(enable_timing=True)
    for e in ev:
        e.record()                       # torch creates the HIP event at its first record
    torch.cuda.synchronize()
    start.record()
    L.bwd(g, events=ev)
    torch.cuda.synchronize()
    for a, b_ in zip(ref, (L.dq, L.dk, L.dv)):
        assert np.array_equal(a, chk.to_np(b_))
    marks = [start] + ev                 # every mark re-recorded after `start`, in launch order
    for e0, e1 in zip(marks, marks[1:]):
        assert e0.elapsed_time(e1) >= 0.0
    assert ev[0].elapsed_time(ev[1]) > 0.0 and ev[2].elapsed_time(ev[3]) > 0.0   # dQ and dK/dV ran


def test_backward_workspace_reused_across_shapes(chk, cases):
    """One workspace serves backward calls of different shapes in turn (its leading
    counters are cleared once and every call leaves them at zero; everything else is
    written before it is read within a call): the results equal those of a workspace
    of their own each time."""
    import sparse_long_context_hga_amd as hga
    names = ["bf16_g8_full_coverage", "bf16_g4_d128_ragged", "bf16_g8_full_coverage"]
    layers = {}
    need = 0
    for name in set(names):
        w, _, _, _, gidx = cases[name]
        L = chk.DeviceLayer(w)
        L.fwd(torch.from_numpy(gidx).cuda())
        L.bwd(torch.from_numpy(gidx).cuda())          # reference, own fresh workspace
        layers[name] = (L, torch.from_numpy(gidx).cuda())
        need = max(need, L.ws.numel())
    torch.cuda.synchronize()
    ref = {n: [chk.to_np(t).copy() for t in (L.dq, L.dk, L.dv)] for n, (L, _) in layers.items()}
    shared = torch.empty(need, dtype=torch.uint8, device="cuda")
    shared[:hga.HGA_BWD_WORKSPACE_CLEAR_BYTES].zero_()   # cleared once: every call leaves it so
    for name in names:
        print(f"case {name} on the shared workspace", flush=True)
        L, g = layers[name]
        for t in (L.dq, L.dk, L.dv):
            t.zero_()
        hga.hga_attend_bwd(L.shape, L.q, L.k, L.v, L.o, L.lse, L.do, L.t_cap, L.t_hist, L.seg_len, g, L.dq, L.dk,
                           L.dv, shared)
        torch.cuda.synchronize()
        for a, b_ in zip(ref[name], (L.dq, L.dk, L.dv)):
            assert np.array_equal(a, chk.to_np(b_)), name
        # the work items' class counts are back at zero for the next call
        assert not shared[:hga.HGA_BWD_WORKSPACE_CLEAR_BYTES].any().item(), name
