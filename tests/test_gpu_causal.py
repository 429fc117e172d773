"""GPU parity of strictly causal routing (hga_route_causal): a block is routed by the
rows of the query block before it (the previous segment's last block for a
segment's first block), everything else as block routing.

  * every unit of the parity layers is accepted against the oracle's causal scores
    (near-tie rule), and the reported scores match;
  * the full chain (causal route -> forward -> backward) matches the oracle on the
    selection the GPU made;
  * the property the variant exists for, on the GPU: steering the queries after
    position p of a block changes the outputs at positions <= p under block
    routing, and leaves them bit-identical under causal routing;
  * the 16K-context layer: every unit accepted, forward on sampled units;
  * two segments through the autograd op with causal routing;
  * hga_forward_causal (summaries, causal routing and attention in one call) bit for
    bit against the separate calls, on every parity layer and the 16K layer.
Expected values come only from the oracle.
"""
import numpy as np
import pytest
import torch

import hga_inputs as hi
from oracle import hga_oracle as ora
from tests.test_gpu_parity import CASES

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def chk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    from tests import hga_check
    import sparse_long_context_hga_amd as hga
    hga.lib()
    return hga_check


def _q_prev(w, seed):
    return hi.prev_query_block(seed=seed, batch=w.batch, n_q_heads=w.n_q_heads, head_dim=w.head_dim,
                               dtype=w.dtype)


def _route_causal_gpu(chk, L, w, q_prev, gs, cs):
    qp = chk.to_dev(q_prev, w.dtype) if w.t_hist > 0 else None
    L.route_causal(qp, chk.to_dev(cs, w.dtype), chk.to_dev(gs, w.dtype))
    torch.cuda.synchronize()
    return L.cidx.cpu().numpy(), L.gidx.cpu().numpy(), L.cscore.cpu().numpy()


def _check_all_units(chk, w, gs, cs, q_prev, cidx, gidx, cscore=None):
    exempt = 0
    for b in range(w.batch):
        for kvh in range(w.n_kv_heads):
            for j in range(w.seg_len // 64):
                exempt += chk.check_route_unit(w, gs, cs, b, kvh, j, cidx[b, kvh, j], gidx[b, kvh, j],
                                               causal=True, q_prev=q_prev)
                if cscore is None:
                    continue
                J = w.t_hist // 64 + j
                if J == 0:
                    continue
                rows = ora.causal_routing_rows(w.q, q_prev, b, kvh, j, w.group_size)
                sig = ora.block_scores(rows, cs[b, kvh, :J])
                for i, c in enumerate(cidx[b, kvh, j]):
                    if c >= 0:
                        assert abs(cscore[b, kvh, j, i] - sig[c]) <= 1e-5 * max(1.0, abs(sig[c]))
                    else:
                        assert cscore[b, kvh, j, i] == -np.inf
    return exempt


@pytest.mark.parametrize("name", list(CASES))
def test_causal_route_accepted(chk, name):
    w = hi.random_layer(name=name, **CASES[name])
    q_prev = _q_prev(w, seed=CASES[name]["seed"])
    print(f"case {name}", flush=True)
    gs, cs = chk.oracle_summaries(w)
    L = chk.DeviceLayer(w)
    cidx, gidx, cscore = _route_causal_gpu(chk, L, w, q_prev, gs, cs)
    exempt = _check_all_units(chk, w, gs, cs, q_prev, cidx, gidx, cscore)
    print(f"near-tie exemptions: {exempt}")


@pytest.mark.parametrize("name", ["bf16_g4_d128_ragged", "bf16_hist0", "f32_g4_d128", "bf16_g8_d128"])
def test_causal_chain_forward_backward(chk, name):
    w = hi.random_layer(name=name, **CASES[name])
    q_prev = _q_prev(w, seed=CASES[name]["seed"])
    print(f"case {name}", flush=True)
    gs, cs = chk.oracle_summaries(w)
    L = chk.DeviceLayer(w)
    T = w.t_hist + w.seg_len
    L.summaries(0, T)
    L.route_causal(chk.to_dev(q_prev, w.dtype) if w.t_hist > 0 else None)
    L.fwd()
    L.bwd()
    torch.cuda.synchronize()
    cidx, gidx = L.cidx.cpu().numpy(), L.gidx.cpu().numpy()
    _check_all_units(chk, w, gs, cs, q_prev, cidx, gidx)
    eo, el = chk.fwd_errors(w, chk.to_np(L.o), chk.to_np(L.lse), gidx)
    errs = chk.bwd_errors(w, chk.to_np(L.dq), chk.to_np(L.dk), chk.to_np(L.dv), gidx)
    print(f"O max-abs {eo:.3e} LSE max-abs {el:.3e} grads rel-L2 {errs}", flush=True)
    assert eo <= chk.TOL_O[w.dtype] and el <= chk.TOL_O[w.dtype]
    chk.assert_grads(errs)


def test_causal_outputs_ignore_later_queries(chk):
    """Steer the queries after position p of block j toward a chunk that block routing
    did not pick: under block routing outputs at positions <= p move (the leak);
    under causal routing they stay bit-identical."""
    kw = dict(CASES["bf16_g4_d128_ragged"])
    kw.update(top_chunks=2, top_groups=9)
    w = hi.random_layer(name="leak", **kw)
    q_prev = _q_prev(w, seed=kw["seed"])
    gs, cs = chk.oracle_summaries(w)
    j, p = 3, 20
    c_blk, _, _ = ora.route(w.q, cs, gs, w.t_hist, w.seg_len, w.top_chunks, w.top_groups, w.group_size)
    q2 = w.q.copy()
    G = w.group_size
    for kvh in range(w.n_kv_heads):
        J = w.t_hist // 64 + j
        target = next(c for c in range(J) if c not in set(c_blk[0, kvh, j].tolist()))
        q2[0, kvh * G:(kvh + 1) * G, 64 * j + p + 1:64 * j + 64] = hi.round_to_bf16(40.0 * cs[0, kvh, target])
    lo = 64 * j + p + 1
    qp = chk.to_dev(q_prev, w.dtype)

    def run(q_np, causal):
        L = chk.DeviceLayer(w)
        L.q.copy_(chk.to_dev(q_np, w.dtype))
        L.summaries(0, w.t_hist + w.seg_len)
        if causal:
            L.route_causal(qp)
        else:
            L.route()
        L.fwd()
        torch.cuda.synchronize()
        return chk.to_np(L.o)

    o_b, o_b2 = run(w.q, False), run(q2, False)
    o_c, o_c2 = run(w.q, True), run(q2, True)
    moved = float(np.max(np.abs(o_b2[:, :, 64 * j:lo] - o_b[:, :, 64 * j:lo])))
    print(f"block routing: outputs before p moved by {moved:.3e}", flush=True)
    assert moved > 1e-2
    np.testing.assert_array_equal(o_c2[:, :, :lo], o_c[:, :, :lo])


def test_causal_qwen3_8b_layer_ctx16k(chk):
    w = hi.qwen_16k()
    q_prev = _q_prev(w, seed=33)
    print(f"workload {w.name} (causal routing)", flush=True)
    L = chk.DeviceLayer(w)
    L.summaries(0, w.t_hist)
    L.summaries(w.t_hist, w.t_hist + w.seg_len)
    L.route_causal(chk.to_dev(q_prev, "bf16"))
    L.fwd()
    torch.cuda.synchronize()
    gs, cs = chk.oracle_summaries(w)
    cidx, gidx = L.cidx.cpu().numpy(), L.gidx.cpu().numpy()
    exempt = _check_all_units(chk, w, gs, cs, q_prev, cidx, gidx)
    print(f"causal route accepted on all units, near-tie exemptions {exempt}", flush=True)
    rng = np.random.default_rng(3)
    units = [(0, int(kvh), int(jj)) for kvh, jj in zip(rng.integers(0, 8, 8), rng.integers(0, 32, 8))]
    eo, el = chk.fwd_errors(w, chk.to_np(L.o), chk.to_np(L.lse), gidx, units=units)
    print(f"O max-abs {eo:.3e} LSE max-abs {el:.3e} on {len(units)} units", flush=True)
    assert eo <= chk.TOL_O["bf16"] and el <= chk.TOL_O["bf16"]


def test_two_segments_causal_through_autograd(chk):
    from sparse_long_context_hga_amd.layer import HGAKVCache, hga_attention
    S, G, Hkv, d = 256, 4, 2, 128
    w = hi.random_layer(seed=41, batch=1, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=d, t_hist=S,
                        seg_len=S, top_chunks=3, top_groups=17, chunk_mean_var=0.5)
    rng = np.random.default_rng(1041)
    q0_np = hi.round_to_bf16(rng.standard_normal(w.q.shape).astype(np.float32))
    print("case two_segments_causal", flush=True)
    dev = lambda x, grad=False: chk.to_dev(x, "bf16").requires_grad_(grad)   # noqa: E731
    cache = HGAKVCache(1, Hkv, d, 2 * S, torch.bfloat16)
    o0, _, g0 = hga_attention(dev(q0_np, True), dev(w.k_cache[:, :, :S]), dev(w.v_cache[:, :, :S]), cache,
                           w.top_chunks, w.top_groups, w.softmax_scale, causal_routing=True)
    cache.commit(S)
    q1 = dev(w.q, True)
    k1 = dev(w.k_cache[:, :, S:2 * S], True)
    v1 = dev(w.v_cache[:, :, S:2 * S], True)
    o1, lse1, gidx1 = hga_attention(q1, k1, v1, cache, w.top_chunks, w.top_groups, w.softmax_scale,
                                    causal_routing=True)
    (o1.float() * chk.to_dev(w.d_o, "f32")).sum().backward()
    torch.cuda.synchronize()
    gs, cs = chk.oracle_summaries(w)
    gsel = gidx1.cpu().numpy()
    q_prev = q0_np[:, :, S - 64:S]                     # segment 0's last block routes segment 1's first
    for kvh in range(Hkv):
        for j in range(S // 64):
            J = S // 64 + j
            rows = ora.causal_routing_rows(w.q, q_prev, 0, kvh, j, G)
            sig = ora.block_scores(rows, cs[0, kvh, :J])
            ocsel = ora.select_topk(sig, list(range(J)), w.top_chunks)
            cidx_row = np.array(ocsel + [-1] * (w.top_chunks - len(ocsel)))
            chk.check_route_unit(w, gs, cs, 0, kvh, j, cidx_row, gsel[0, kvh, j], causal=True, q_prev=q_prev)
    eo, el = chk.fwd_errors(w, chk.to_np(o1), chk.to_np(lse1), gsel)
    errs = chk.bwd_errors(w, chk.to_np(q1.grad), chk.to_np(k1.grad), chk.to_np(v1.grad), gsel)
    print(f"O max-abs {eo:.3e} LSE max-abs {el:.3e} grad rel-L2 {errs}", flush=True)
    assert eo <= chk.TOL_O["bf16"] and el <= chk.TOL_O["bf16"]
    chk.assert_grads(errs)
    # a cache filled without causal routing cannot route the next segment causally
    cache2 = HGAKVCache(1, Hkv, d, 2 * S, torch.bfloat16)
    cache2.length = S
    with pytest.raises(ValueError):
        hga_attention(q1, k1, v1, cache2, w.top_chunks, w.top_groups, causal_routing=True)


def _fused_vs_separate(chk, w, q_prev):
    qp = chk.to_dev(q_prev, w.dtype) if w.t_hist > 0 else None
    A = chk.DeviceLayer(w)
    A.summaries(0, w.t_hist + w.seg_len)
    A.route_causal(qp)
    A.fwd()
    B = chk.DeviceLayer(w)
    B.summaries(0, w.t_hist)
    B.forward_causal(qp)
    torch.cuda.synchronize()
    for field in ("gsum", "csum", "cidx", "gidx", "o", "lse"):
        assert torch.equal(getattr(A, field), getattr(B, field)), f"hga_forward_causal: {field} differs"


@pytest.mark.parametrize("name", list(CASES))
def test_forward_causal_matches_separate_calls(chk, name):
    w = hi.random_layer(name=name, **CASES[name])
    print(f"case {name}", flush=True)
    _fused_vs_separate(chk, w, _q_prev(w, seed=CASES[name]["seed"]))


def test_forward_causal_qwen3_8b_layer_ctx16k(chk):
    w = hi.qwen_16k()
    print(f"workload {w.name} (hga_forward_causal)", flush=True)
    _fused_vs_separate(chk, w, _q_prev(w, seed=33))
