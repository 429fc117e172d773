"""GPU parity on the five named workloads, every unit (seeded synthetic stand-ins
for the pages' Qwen3-8B / PG19 setting: 32 query / 8 KV heads, head_dim 128,
2,048-token segments, 64-token chunks, 8-token groups, top-16 chunks / top-64
groups).

  tiny_f32_1k            one head, head_dim 64, one 1,024-token segment, fp32, fwd;
                         the full-coverage budget must equal dense causal attention
  qwen3_8b_layer_ctx4k   2,048 history + 2,048 active, bf16, fwd+bwd
  qwen3_8b_layer_ctx16k  14,336 history + 2,048 active, block-structured keys
  rollout 131,072        64 successive 2,048-token segments against a growing
                         history held on the GPU, fwd only: one test per segment
  planted 8 x 32,768     last segment fwd+bwd; planted-chunk recall

For every workload and every unit (sequence, KV head, query block):
  * the summaries are bit-exact;
  * the GPU's selection is accepted by the near-tie rule against the oracle's
    scores (exemptions recorded and bounded);
  * O and LSE (and, with a backward, dQ, dK, dV over whole tensors and per 64-row
    block / chunk) of the library given the oracle's selection match the oracle;
  * on every unit where the GPU chose what the oracle chose, the chained forward
    (GPU routing) is bit-identical to the forward given the oracle's selection.
Inputs flow one way only: the oracle's selection is given to the library, never
the reverse.
"""
import types

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


def _full_layer_check(chk, w, backward=True):
    print(f"workload {w.name}", flush=True)
    L = chk.DeviceLayer(w)
    L.summaries(0, w.t_hist)                      # history: built once
    L.summaries(w.t_hist, w.t_hist + w.seg_len)   # active segment
    L.route()
    L.fwd()                                       # chained: the GPU's own selection
    torch.cuda.synchronize()
    gs, cs = chk.oracle_summaries(w)
    T = w.t_hist + w.seg_len
    np.testing.assert_array_equal(chk.to_np(L.gsum)[:, :, :T // 8], gs[:, :, :T // 8])
    np.testing.assert_array_equal(chk.to_np(L.csum)[:, :, :T // 64], cs[:, :, :T // 64])
    cidx, gidx = L.cidx.cpu().numpy(), L.gidx.cpu().numpy()
    o_chain, lse_chain = chk.to_np(L.o), chk.to_np(L.lse)
    ocidx, ogidx, tables = chk.oracle_route(w, gs, cs)
    chk.accept_all_units(w, gs, cs, cidx, gidx, w.name, ocidx, tables)
    og = torch.from_numpy(ogidx).cuda()
    L.fwd(og)
    if backward:
        L.bwd(og)
    torch.cuda.synchronize()
    o, lse = chk.to_np(L.o), chk.to_np(L.lse)
    n_same = chk.chain_matches(w, gidx, ogidx, o_chain, lse_chain, o, lse)
    eo, el = chk.fwd_errors(w, o, lse, ogidx)
    print(f"O max-abs {eo:.3e}  LSE max-abs {el:.3e} (every unit); chained forward bit-identical on "
          f"{n_same} units with the oracle's selection", flush=True)
    assert eo <= chk.TOL_O[w.dtype] and el <= chk.TOL_O[w.dtype]
    if backward:
        errs = chk.bwd_errors(w, chk.to_np(L.dq), chk.to_np(L.dk), chk.to_np(L.dv), ogidx)
        print(f"grad rel-L2 {errs}", flush=True)
        chk.assert_grads(errs)
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


# ---------------------------------------------------------------- 131K rollout
ROLLOUT_SEGMENTS = hi.ROLLOUT_TOKENS // hi.ROLLOUT_SEG


@pytest.fixture(scope="module")
def rollout(chk):
    """The 131,072-token rollout run once on the GPU: 64 segments, each writing its
    K/V, building its summaries, routing over every earlier segment and itself and
    attending.  Keeps each segment's selection and outputs for the per-segment tests."""
    import sparse_long_context_hga_amd as hga
    S, Hq, Hkv, d, T = hi.ROLLOUT_SEG, 32, 8, 128, hi.ROLLOUT_TOKENS
    shape = hga.make_shape(1, Hq, Hkv, d, 16, 64, "bf16", 1.0 / np.sqrt(d))
    kc = torch.zeros(1, Hkv, T, d, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    gsum = torch.zeros(1, Hkv, T // 8, d, dtype=torch.bfloat16, device="cuda")
    csum = torch.zeros(1, Hkv, T // 64, d, dtype=torch.bfloat16, device="cuda")
    nb = S // 64
    k_host = np.zeros((1, Hkv, T, d), np.float32)
    v_host = np.zeros((1, Hkv, T, d), np.float32)
    R = types.SimpleNamespace(shape=shape, kc=kc, vc=vc, k_host=k_host, v_host=v_host, q_host=[], q_dev=[],
                              cidx=[], gidx=[], o=[], lse=[], S=S, T=T, Hq=Hq, Hkv=Hkv, d=d)
    for s in range(ROLLOUT_SEGMENTS):
        q, k, v = hi.rollout_segment(s)
        k_host[:, :, s * S:(s + 1) * S] = k
        v_host[:, :, s * S:(s + 1) * S] = v
        kc[:, :, s * S:(s + 1) * S] = torch.from_numpy(k).to(torch.bfloat16).cuda()
        vc[:, :, s * S:(s + 1) * S] = torch.from_numpy(v).to(torch.bfloat16).cuda()
        qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
        cidx = torch.empty(1, Hkv, nb, 16, dtype=torch.int32, device="cuda")
        gidx = torch.empty(1, Hkv, nb, 64, dtype=torch.int32, device="cuda")
        o = torch.empty(1, Hq, S, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(1, Hq, S, dtype=torch.float32, device="cuda")
        hga.hga_build_summaries(shape, kc, T, s * S, (s + 1) * S, gsum, csum)
        hga.hga_route(shape, qd, csum, gsum, T, s * S, S, cidx, gidx)
        hga.hga_attend_fwd(shape, qd, kc, vc, T, s * S, S, gidx, o, lse)
        R.q_host.append(q)
        R.q_dev.append(qd)
        R.cidx.append(cidx)
        R.gidx.append(gidx)
        R.o.append(o)
        R.lse.append(lse)
        if s % 16 == 15:
            torch.cuda.synchronize()
            print(f"rollout: {s + 1} segments done", flush=True)
    torch.cuda.synchronize()
    R.gs = np.zeros((1, Hkv, T // 8, d), np.float32)
    R.cs = np.zeros((1, Hkv, T // 64, d), np.float32)
    ora.build_summaries(k_host, 0, T, "bf16", R.gs, R.cs)
    np.testing.assert_array_equal(gsum.float().cpu().numpy(), R.gs)
    np.testing.assert_array_equal(csum.float().cpu().numpy(), R.cs)
    print("rollout: summaries of all 131,072 tokens bit-exact", flush=True)
    return R


@pytest.mark.parametrize("s", range(ROLLOUT_SEGMENTS))
def test_rollout_131k_segment(chk, rollout, s):
    """Segment s of the rollout (history s x 2,048 tokens): routing accepted on every
    unit, O and LSE on every unit."""
    import sparse_long_context_hga_amd as hga
    R = rollout
    S, T = R.S, R.T
    w = hi.Workload(name=f"rollout_131k_s{s}", batch=1, n_q_heads=R.Hq, n_kv_heads=R.Hkv, head_dim=R.d,
                    t_hist=s * S, seg_len=S, t_cap=T, top_chunks=16, top_groups=64, dtype="bf16",
                    softmax_scale=1.0 / np.sqrt(R.d), backward=False, q=R.q_host[s], k_cache=R.k_host,
                    v_cache=R.v_host, d_o=None)
    print(f"rollout segment {s}: t_hist={w.t_hist}", flush=True)
    cidx, gidx = R.cidx[s].cpu().numpy(), R.gidx[s].cpu().numpy()
    ocidx, ogidx, tables = chk.oracle_route(w, R.gs, R.cs)
    chk.accept_all_units(w, R.gs, R.cs, cidx, gidx, w.name, ocidx, tables)
    o = torch.empty_like(R.o[s])
    lse = torch.empty_like(R.lse[s])
    hga.hga_attend_fwd(R.shape, R.q_dev[s], R.kc, R.vc, T, s * S, S, torch.from_numpy(ogidx).cuda(), o, lse)
    torch.cuda.synchronize()
    o_np, lse_np = chk.to_np(o), chk.to_np(lse)
    n_same = chk.chain_matches(w, gidx, ogidx, chk.to_np(R.o[s]), chk.to_np(R.lse[s]), o_np, lse_np)
    eo, el = chk.fwd_errors(w, o_np, lse_np, ogidx)
    print(f"segment {s}: O max-abs {eo:.3e} LSE max-abs {el:.3e} on all {S // 64 * R.Hkv} units; chained "
          f"forward bit-identical on {n_same}", flush=True)
    assert eo <= chk.TOL_O["bf16"] and el <= chk.TOL_O["bf16"]


# ---------------------------------------------------------------- planted batch
@pytest.fixture(scope="module")
def planted(chk):
    """Batch 8 x 32,768 with planted chunks: the GPU's own step (summaries, route,
    forward, backward) and the oracle's summaries and selection."""
    w = hi.planted_batch()
    print(f"workload {w.name}", flush=True)
    L = chk.DeviceLayer(w)
    L.summaries(0, w.t_hist)
    L.step()
    torch.cuda.synchronize()
    P = types.SimpleNamespace(w=w, L=L, cidx=L.cidx.cpu().numpy(), gidx=L.gidx.cpu().numpy(),
                              o_chain=chk.to_np(L.o), lse_chain=chk.to_np(L.lse))
    P.gs = np.zeros(L.gsum.shape, np.float32)
    P.cs = np.zeros(L.csum.shape, np.float32)
    ora.build_summaries(w.k_cache, 0, w.t_hist + w.seg_len, "bf16", P.gs, P.cs)
    np.testing.assert_array_equal(chk.to_np(L.gsum), P.gs)
    np.testing.assert_array_equal(chk.to_np(L.csum), P.cs)
    P.ocidx, P.ogidx, P.tables = chk.oracle_route(w, P.gs, P.cs)
    print("planted: summaries bit-exact, oracle selection done", flush=True)
    return P


def test_planted_b8_ctx32k_recall(chk, planted):
    """Every unit of every sequence selects all 4 planted chunks and their 32 groups."""
    w, P = planted.w, planted
    nb = w.seg_len // 64
    for b in range(w.batch):
        pc = set(int(c) for c in w.extra["planted_chunks"][b])
        pg = {8 * c + u for c in pc for u in range(8)}
        for kvh in range(w.n_kv_heads):
            for j in range(nb):
                assert pc <= set(int(c) for c in P.cidx[b, kvh, j]), (b, kvh, j)
                assert pg <= set(int(g) for g in P.gidx[b, kvh, j]), (b, kvh, j)
    print("planted recall 1.0 on all units", flush=True)


def test_planted_with_decoys_route(chk):
    """Direction control on the GPU: 2 sequences of 8,192 tokens (32/8/128, bf16)
    with 4 planted chunks and 4 decoy chunks (keys at cosine -0.9 with the planted
    direction) each.  The fused routing + attention call's selection is accepted
    against the oracle on every unit and holds every planted chunk and group."""
    w = hi.planted_batch(batch=2, t_total=8192, seg_len=2048, seed=56, n_decoys=4)
    print(f"workload {w.name} with decoys", flush=True)
    L = chk.DeviceLayer(w)
    L.summaries(0, w.t_hist)
    L.forward()
    torch.cuda.synchronize()
    cidx, gidx = L.cidx.cpu().numpy(), L.gidx.cpu().numpy()
    gs, cs = chk.oracle_summaries(w)
    ocidx, _, tables = chk.oracle_route(w, gs, cs)
    chk.accept_all_units(w, gs, cs, cidx, gidx, "planted_decoys", ocidx, tables)
    for b in range(w.batch):
        pc = set(int(c) for c in w.extra["planted_chunks"][b])
        pg = {8 * c + u for c in pc for u in range(8)}
        for kvh in range(w.n_kv_heads):
            for j in range(w.seg_len // 64):
                assert pc <= set(int(c) for c in cidx[b, kvh, j]), (b, kvh, j)
                assert pg <= set(int(g) for g in gidx[b, kvh, j]), (b, kvh, j)
    print("planted recall 1.0 with decoys present", flush=True)


def test_planted_b8_ctx32k_route(chk, planted):
    P = planted
    chk.accept_all_units(P.w, P.gs, P.cs, P.cidx, P.gidx, P.w.name, P.ocidx, P.tables)


def test_planted_b8_ctx32k_forward(chk, planted):
    P, w = planted, planted.w
    P.L.fwd(torch.from_numpy(P.ogidx).cuda())
    torch.cuda.synchronize()
    o, lse = chk.to_np(P.L.o), chk.to_np(P.L.lse)
    n_same = chk.chain_matches(w, P.gidx, P.ogidx, P.o_chain, P.lse_chain, o, lse)
    eo, el = chk.fwd_errors(w, o, lse, P.ogidx)
    print(f"O max-abs {eo:.3e}  LSE max-abs {el:.3e} on all {w.batch * w.n_kv_heads * w.seg_len // 64} units; "
          f"chained forward bit-identical on {n_same}", flush=True)
    assert eo <= chk.TOL_O["bf16"] and el <= chk.TOL_O["bf16"]


def test_planted_b8_ctx32k_backward(chk, planted):
    P, w = planted, planted.w
    og = torch.from_numpy(P.ogidx).cuda()
    P.L.fwd(og)
    P.L.bwd(og)
    torch.cuda.synchronize()
    errs = chk.bwd_errors(w, chk.to_np(P.L.dq), chk.to_np(P.L.dk), chk.to_np(P.L.dv), P.ogidx)
    print(f"grad rel-L2 {errs} (every unit and chunk)", flush=True)
    chk.assert_grads(errs)
