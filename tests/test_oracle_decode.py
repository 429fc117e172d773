"""Pins for the oracle's generation path (reading R-decode): one new token per
sequence, routed by its own query heads, attending the selected groups plus its
own chunk up to itself; the summaries of a chunk are built when its last token
arrives.

Checked against: dense causal attention written out directly (full-coverage
budget), attention over the own-chunk window alone (zero budget), the
mean-logit identity and exhaustive subset enumeration for the selection, the
bulk summary build for the incremental updates, invariance to everything after
the token, and the convex-hull / LSE bounds.
"""
import itertools

import numpy as np

import hga_inputs as hi
from oracle import hga_oracle as ora


def _summaries(w, upto=None):
    B, H, T, d = w.k_cache.shape
    gs = np.zeros((B, H, T // 8, d), np.float32)
    cs = np.zeros((B, H, T // 64, d), np.float32)
    ora.build_summaries(w.k_cache, 0, T if upto is None else upto, w.dtype, gs, cs)
    return gs, cs


def _dense_window(q_rows, K, V, scale, lo, hi_):
    """Softmax attention of rows [G, d] over positions lo .. hi_ (inclusive), float64."""
    k = K[lo:hi_ + 1].astype(np.float64)
    v = V[lo:hi_ + 1].astype(np.float64)
    lg = scale * (q_rows.astype(np.float64) @ k.T)
    m = lg.max(1, keepdims=True)
    e = np.exp(lg - m)
    return (e / e.sum(1, keepdims=True)) @ v, (m[:, 0] + np.log(e.sum(1)))


def _layer(**kw):
    base = dict(seed=61, batch=3, n_q_heads=4, n_kv_heads=2, head_dim=32, t_cap=384, pos=[100, 255, 319],
                top_chunks=3, top_groups=7, dtype="f32")
    base.update(kw)
    return hi.decode_batch(**base)


def _run(w, gs, cs, kc=None, kg=None):
    kc = w.top_chunks if kc is None else kc
    kg = w.top_groups if kg is None else kg
    cidx, gidx, tables = ora.decode_route(w.q, cs, gs, w.pos, kc, kg, w.group_size)
    o, lse = ora.decode_attend(w.q, w.k_cache, w.v_cache, w.pos, gidx, w.softmax_scale, w.group_size)
    return cidx, gidx, o, lse, tables


def test_full_coverage_is_dense_causal_attention():
    w = _layer()
    gs, cs = _summaries(w)
    cidx, gidx, o, lse, _ = _run(w, gs, cs, kc=8, kg=64)
    G = w.group_size
    for b in range(w.batch):
        J = int(w.pos[b]) // 64
        assert cidx[b, 0, :J].tolist() == list(range(J)) and np.all(cidx[b, 0, J:] == -1)
        for kvh in range(2):
            od, ld = _dense_window(w.q[b, kvh * G:(kvh + 1) * G], w.k_cache[b, kvh], w.v_cache[b, kvh],
                                   w.softmax_scale, 0, int(w.pos[b]))
            np.testing.assert_allclose(o[b, kvh * G:(kvh + 1) * G], od, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, kvh * G:(kvh + 1) * G], ld, rtol=0, atol=1e-12)


def test_zero_budget_is_own_chunk_window():
    w = _layer()
    gs, cs = _summaries(w)
    cidx, gidx, o, lse, _ = _run(w, gs, cs, kc=0, kg=0)
    G = w.group_size
    for b in range(w.batch):
        p = int(w.pos[b])
        for kvh in range(2):
            od, ld = _dense_window(w.q[b, kvh * G:(kvh + 1) * G], w.k_cache[b, kvh], w.v_cache[b, kvh],
                                   w.softmax_scale, 64 * (p // 64), p)
            np.testing.assert_allclose(o[b, kvh * G:(kvh + 1) * G], od, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, kvh * G:(kvh + 1) * G], ld, rtol=0, atol=1e-12)


def _brute_topk(scores, ids, k):
    k = min(k, len(ids))
    found = []
    for sub in itertools.combinations(range(len(ids)), k):
        inside = set(sub)
        if all((scores[x] > scores[y]) or (scores[x] == scores[y] and ids[x] < ids[y])
               for x in inside for y in range(len(ids)) if y not in inside):
            found.append(sorted(ids[x] for x in sub))
    assert len(found) == 1
    return found[0]


def test_route_scores_and_selection_by_brute_force():
    w = _layer(seed=62, batch=2, n_q_heads=4, n_kv_heads=2, head_dim=16, t_cap=512, pos=[300, 450],
               top_chunks=3, top_groups=5)
    gs, cs = _summaries(w)
    kk = w.k_cache.astype(np.float64)
    for b in range(2):
        p = int(w.pos[b])
        J = p // 64
        for kvh in range(2):
            c_sel, g_sel, sig, gids, tau = ora.decode_route_unit(w.q, cs, gs, p, b, kvh, 3, 5, 2)
            rows = w.q[b, 2 * kvh:2 * kvh + 2].astype(np.float64)
            kb = kk[b, kvh]
            brute = np.array([max(float(np.mean(kb[64 * c:64 * c + 64] @ r)) for r in rows) for c in range(J)])
            assert np.max(np.abs(sig - brute)) <= 1e-5 * (1 + np.max(np.abs(brute)))
            assert c_sel == _brute_topk(sig, list(range(J)), 3)
            gbrute = np.array([max(float(np.mean(kb[8 * g:8 * g + 8] @ r)) for r in rows) for g in gids])
            assert np.max(np.abs(tau - gbrute)) <= 1e-5 * (1 + np.max(np.abs(gbrute)))
            assert g_sel == _brute_topk(tau, gids, 5)


def test_incremental_summaries_equal_the_bulk_build():
    """Generating positions one at a time (sequence 1 seven tokens behind) and
    updating the summaries as chunks complete gives the bulk tables bit-exactly;
    a chunk that has not completed is never written."""
    w = _layer(seed=63, batch=2, n_q_heads=2, n_kv_heads=1, head_dim=16, t_cap=320, pos=[0, 0], dtype="bf16")
    B, H, T, d = w.k_cache.shape
    gs = np.zeros((B, H, T // 8, d), np.float32)
    cs = np.zeros((B, H, T // 64, d), np.float32)
    for p in range(0, 263):
        ora.decode_summaries(w.k_cache, np.array([p, p - 7]), "bf16", gs, cs)
    ref_g, ref_c = _summaries(w, upto=256)
    np.testing.assert_array_equal(gs, ref_g)
    np.testing.assert_array_equal(cs, ref_c)
    assert not cs[:, :, 4:].any() and not gs[:, :, 32:].any()


def test_nothing_after_the_token_matters_and_idle_slots():
    w = _layer(seed=64, pos=[100, 255, -1])
    gs, cs = _summaries(w)
    cidx, gidx, o, lse, _ = _run(w, gs, cs)
    assert np.all(cidx[2] == -1) and np.all(gidx[2] == -1)
    assert np.all(o[2] == 0) and np.all(lse[2] == -np.inf)
    w2 = _layer(seed=64, pos=[100, 255, -1])
    rng = np.random.default_rng(9)
    for b in range(2):
        p = int(w.pos[b])
        w2.k_cache[b, :, p + 1:] = rng.standard_normal(w2.k_cache[b, :, p + 1:].shape) * 3
        w2.v_cache[b, :, p + 1:] = rng.standard_normal(w2.v_cache[b, :, p + 1:].shape) * 3
    gs2, cs2 = _summaries(w2)
    cidx2, gidx2, o2, lse2, _ = _run(w2, gs2, cs2)
    np.testing.assert_array_equal(cidx2, cidx)
    np.testing.assert_array_equal(gidx2, gidx)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(lse2, lse)


def test_constant_values_and_lse_bound():
    w = _layer(seed=65)
    c = np.random.default_rng(2).standard_normal((w.batch, 2, 1, 32)).astype(np.float32)
    w.v_cache[:] = c
    gs, cs = _summaries(w)
    cidx, gidx, o, lse, _ = _run(w, gs, cs)
    G = w.group_size
    for b in range(w.batch):
        for kvh in range(2):
            np.testing.assert_allclose(o[b, kvh * G:(kvh + 1) * G], np.broadcast_to(c[b, kvh], (G, 32)),
                                       rtol=0, atol=1e-12)
            tok = ora.decode_key_tokens(gidx[b, kvh], int(w.pos[b]))
            lg = w.softmax_scale * (w.q[b, kvh * G:(kvh + 1) * G].astype(np.float64) @
                                    w.k_cache[b, kvh][tok].astype(np.float64).T)
            assert np.all(lse[b, kvh * G:(kvh + 1) * G] >= lg.max(1) - 1e-12)
            assert np.all(lse[b, kvh * G:(kvh + 1) * G] <= lg.max(1) + np.log(len(tok)) + 1e-12)
