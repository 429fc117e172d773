"""GPU parity on the five named workloads (seeded synthetic stand-ins for the
pages' Qwen3-8B / PG19 setting: 32 query / 8 KV heads, head_dim 128, 2,048-token
segments, 64-token chunks, 8-token groups, top-16 chunks / top-64 groups).

  tiny_f32_1k            one head, head_dim 64, one 1,024-token segment, fp32, fwd:
                         every unit compared; the full-coverage budget must equal
                         dense causal attention
  qwen3_8b_layer_ctx4k   2,048 history + 2,048 active, bf16, fwd+bwd: every unit
  qwen3_8b_layer_ctx16k  14,336 history + 2,048 active, block-structured keys:
                         every unit
  rollout 131,072        64 successive 2,048-token segments against a growing
                         history held on the GPU, fwd only: sampled segments/units
  planted 8 x 32,768     last segment fwd+bwd; planted-chunk recall on every unit,
                         sampled units against the oracle

Routing is checked with the near-tie acceptance rule; attention and gradients on
the oracle's own selection (given to the library as input) and, for the full
chain, on units where both selections agree.
"""
import numpy as np
import pytest
import torch

import hga_inputs as hi
from oracle import hga_oracle as ora

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def chk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    from tests import hga_check
    import sparse_long_context_hga_amd as hga
    hga.lib()
    return hga_check


def _oracle_gidx(w, gs, cs, units):
    """Group selection computed by the oracle for the given units (-1 elsewhere)."""
    g = np.full((w.batch, w.n_kv_heads, w.seg_len // 64, w.top_groups), -1, np.int32)
    for (b, kvh, j) in units:
        sel = ora.route_unit(w.q, cs, gs, w.t_hist, b, kvh, j, w.top_chunks, w.top_groups, w.group_size)[1]
        g[b, kvh, j, :len(sel)] = sel
    return g


def _full_layer_check(chk, w, backward=True):
    print(f"workload {w.name}", flush=True)
    L = chk.DeviceLayer(w)
    L.summaries(0, w.t_hist)                      # history: built once
    L.summaries(w.t_hist, w.t_hist + w.seg_len)   # active segment
    L.route()
    torch.cuda.synchronize()
    gs, cs = chk.oracle_summaries(w)
    T = w.t_hist + w.seg_len
    np.testing.assert_array_equal(chk.to_np(L.gsum)[:, :, :T // 8], gs[:, :, :T // 8])
    np.testing.assert_array_equal(chk.to_np(L.csum)[:, :, :T // 64], cs[:, :, :T // 64])
    cidx, gidx = L.cidx.cpu().numpy(), L.gidx.cpu().numpy()
    exempt = 0
    for b in range(w.batch):
        for kvh in range(w.n_kv_heads):
            for j in range(w.seg_len // 64):
                exempt += chk.check_route_unit(w, gs, cs, b, kvh, j, cidx[b, kvh, j], gidx[b, kvh, j])
    print(f"route accepted on all units, near-tie exemptions {exempt}", flush=True)
    _, ogidx, _ = chk.oracle_route(w, gs, cs)
    og = torch.from_numpy(ogidx).cuda()
    L.fwd(og)
    if backward:
        L.bwd(og)
    torch.cuda.synchronize()
    eo, el = chk.fwd_errors(w, chk.to_np(L.o), chk.to_np(L.lse), ogidx)
    print(f"O max-abs {eo:.3e}  LSE max-abs {el:.3e}", flush=True)
    assert eo <= chk.TOL_O[w.dtype] and el <= chk.TOL_O[w.dtype]
    if backward:
        errs = chk.bwd_errors(w, chk.to_np(L.dq), chk.to_np(L.dk), chk.to_np(L.dv), ogidx)
        print(f"grad rel-L2 {errs}", flush=True)
        assert all(v <= chk.TOL_GRAD_REL_L2 for v in errs.values())
    return L, ogidx


def test_tiny_f32_1k(chk):
    _full_layer_check(chk, hi.tiny_f32(), backward=False)


def test_tiny_f32_1k_full_coverage_is_dense(chk):
    w = hi.tiny_f32(full_coverage=True)
    L, ogidx = _full_layer_check(chk, w, backward=False)
    # with every chunk and group selected the layer is dense causal attention
    q = w.q[0, 0].astype(np.float64)
    k = w.k_cache[0, 0, :1024].astype(np.float64)
    v = w.v_cache[0, 0, :1024].astype(np.float64)
    lg = (q @ k.T) * w.softmax_scale
    lg[np.triu_indices(1024, 1)] = -np.inf
    p = np.exp(lg - lg.max(1, keepdims=True))
    dense = (p / p.sum(1, keepdims=True)) @ v
    assert np.max(np.abs(chk.to_np(L.o)[0, 0] - dense)) <= 1e-4


def test_qwen3_8b_layer_ctx4k(chk):
    _full_layer_check(chk, hi.qwen_2k_hist())


def test_qwen3_8b_layer_ctx16k(chk):
    _full_layer_check(chk, hi.qwen_16k())


def test_rollout_131k(chk):
    """64 segments of 2,048 tokens, each routed against all earlier ones (history on the GPU)."""
    import sparse_long_context_hga_amd as hga
    S, n_seg, Hq, Hkv, d = hi.ROLLOUT_SEG, hi.ROLLOUT_TOKENS // hi.ROLLOUT_SEG, 32, 8, 128
    T = hi.ROLLOUT_TOKENS
    shape = hga.make_shape(1, Hq, Hkv, d, 16, 64, "bf16", 1.0 / np.sqrt(d))
    kc = torch.zeros(1, Hkv, T, d, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    gsum = torch.zeros(1, Hkv, T // 8, d, dtype=torch.bfloat16, device="cuda")
    csum = torch.zeros(1, Hkv, T // 64, d, dtype=torch.bfloat16, device="cuda")
    nb = S // 64
    cidx = torch.empty(1, Hkv, nb, 16, dtype=torch.int32, device="cuda")
    gidx = torch.empty(1, Hkv, nb, 64, dtype=torch.int32, device="cuda")
    o = torch.empty(1, Hq, S, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, Hq, S, dtype=torch.float32, device="cuda")
    k_host = np.zeros((1, Hkv, T, d), np.float32)
    v_host = np.zeros((1, Hkv, T, d), np.float32)
    sampled = {0: None, 1: None, 31: None, 63: None}
    for s in range(n_seg):
        q, k, v = hi.rollout_segment(s)
        k_host[:, :, s * S:(s + 1) * S] = k
        v_host[:, :, s * S:(s + 1) * S] = v
        kc[:, :, s * S:(s + 1) * S] = torch.from_numpy(k).to(torch.bfloat16).cuda()
        vc[:, :, s * S:(s + 1) * S] = torch.from_numpy(v).to(torch.bfloat16).cuda()
        qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
        hga.hga_build_summaries(shape, kc, T, s * S, (s + 1) * S, gsum, csum)
        hga.hga_route(shape, qd, csum, gsum, T, s * S, S, cidx, gidx)
        hga.hga_attend_fwd(shape, qd, kc, vc, T, s * S, S, gidx, o, lse)
        if s in sampled:
            torch.cuda.synchronize()
            sampled[s] = (q, gidx.cpu().numpy().copy(), o.float().cpu().numpy(), lse.cpu().numpy(),
                          cidx.cpu().numpy().copy())
            print(f"rollout segment {s} done", flush=True)
    torch.cuda.synchronize()
    gs = np.zeros((1, Hkv, T // 8, d), np.float32)
    cs = np.zeros((1, Hkv, T // 64, d), np.float32)
    ora.build_summaries(k_host, 0, T, "bf16", gs, cs)
    np.testing.assert_array_equal(gsum.float().cpu().numpy(), gs)
    np.testing.assert_array_equal(csum.float().cpu().numpy(), cs)
    rng = np.random.default_rng(0)
    for s, (q, g_gpu, o_gpu, l_gpu, c_gpu) in sampled.items():
        w = hi.Workload(name=f"rollout_s{s}", batch=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                        t_hist=s * S, seg_len=S, t_cap=T, top_chunks=16, top_groups=64, dtype="bf16",
                        softmax_scale=1.0 / np.sqrt(d), backward=False, q=q, k_cache=k_host,
                        v_cache=v_host, d_o=None)
        units = [(0, int(kvh), int(j)) for kvh, j in zip(rng.integers(0, Hkv, 6), rng.integers(0, nb, 6))]
        agree = []
        og = _oracle_gidx(w, gs, cs, units)
        for (b, kvh, j) in units:
            chk.check_route_unit(w, gs, cs, b, kvh, j, c_gpu[b, kvh, j], g_gpu[b, kvh, j])
            if np.array_equal(g_gpu[b, kvh, j], og[b, kvh, j]):
                agree.append((b, kvh, j))
        assert len(agree) >= len(units) - 1
        eo, el = chk.fwd_errors(w, o_gpu, l_gpu, og, units=agree)
        print(f"segment {s}: {len(agree)}/{len(units)} sampled units identical selection, "
              f"O max-abs {eo:.3e} LSE max-abs {el:.3e}", flush=True)
        assert eo <= chk.TOL_O["bf16"] and el <= chk.TOL_O["bf16"]


def test_planted_b8_ctx32k(chk):
    w = hi.planted_batch()
    print(f"workload {w.name}", flush=True)
    L = chk.DeviceLayer(w)
    L.summaries(0, w.t_hist)
    L.step()
    torch.cuda.synchronize()
    cidx, gidx = L.cidx.cpu().numpy(), L.gidx.cpu().numpy()
    planted = w.extra["planted_chunks"]
    nb = w.seg_len // 64
    for b in range(w.batch):                         # recall = 1 on every unit
        pc = set(int(c) for c in planted[b])
        pg = {8 * c + u for c in pc for u in range(8)}
        for kvh in range(w.n_kv_heads):
            for j in range(nb):
                assert pc <= set(int(c) for c in cidx[b, kvh, j]), (b, kvh, j)
                assert pg <= set(int(g) for g in gidx[b, kvh, j]), (b, kvh, j)
    print("planted recall 1.0 on all units", flush=True)
    gs = np.zeros(L.gsum.shape, np.float32)
    cs = np.zeros(L.csum.shape, np.float32)
    ora.build_summaries(w.k_cache, 0, w.t_hist + w.seg_len, "bf16", gs, cs)
    rng = np.random.default_rng(1)
    units = [(int(b), int(kvh), int(j)) for b, kvh, j in
             zip(rng.integers(0, w.batch, 12), rng.integers(0, w.n_kv_heads, 12), rng.integers(0, nb, 12))]
    # the oracle's own selection for the sampled units and every block attending their chunks
    need = sorted({(b, kvh, jj) for (b, kvh, j) in units for jj in range(j, nb)})
    og = _oracle_gidx(w, gs, cs, need)
    agree = []
    for (b, kvh, j) in units:
        chk.check_route_unit(w, gs, cs, b, kvh, j, cidx[b, kvh, j], gidx[b, kvh, j])
        if np.array_equal(gidx[b, kvh, j], og[b, kvh, j]):
            agree.append((b, kvh, j))
    assert len(agree) >= len(units) - 1
    eo, el = chk.fwd_errors(w, chk.to_np(L.o), chk.to_np(L.lse), og, units=agree)
    print(f"O max-abs {eo:.3e}  LSE max-abs {el:.3e} on {len(agree)} units", flush=True)
    assert eo <= chk.TOL_O["bf16"] and el <= chk.TOL_O["bf16"]
    # gradients: dQ of the sampled units and dK/dV of sampled active chunks whose every
    # attending block selected exactly what the oracle selects
    chunks = [(b, kvh, cc) for (b, kvh, cc) in units
              if all(np.array_equal(gidx[b, kvh, jj], og[b, kvh, jj]) for jj in range(cc, nb))]
    assert chunks
    errs = chk.bwd_errors(w, chk.to_np(L.dq), chk.to_np(L.dk), chk.to_np(L.dv), og, units=agree, chunks=chunks)
    print(f"grad rel-L2 {errs} ({len(chunks)} chunks)", flush=True)
    assert all(v <= chk.TOL_GRAD_REL_L2 for v in errs.values())
