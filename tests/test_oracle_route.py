"""Pins for the oracle's routing (readings R-score, R-cand, R-group, R-topk).

Checked against: the linearity identity (a summary score equals the mean raw
logit over the chunk's tokens, computed without ever forming a summary),
exhaustive k-subset enumeration on tiny inputs, and the planted-chunk recall
that the planted workload is built to guarantee.
"""
import itertools

import numpy as np
import pytest

import hga_inputs as hi
from oracle import hga_oracle as ora


def _summaries(w):
    B, H, T, d = w.k_cache.shape
    gs = np.zeros((B, H, T // 8, d), np.float32)
    cs = np.zeros((B, H, T // 64, d), np.float32)
    ora.build_summaries(w.k_cache, 0, w.t_hist + w.seg_len, w.dtype, gs, cs)
    return gs, cs


def test_chunk_scores_equal_mean_logit_over_chunk_tokens():
    w = hi.random_layer(seed=5, batch=1, n_q_heads=4, n_kv_heads=2, head_dim=32, t_hist=512,
                        seg_len=256, top_chunks=3, top_groups=10, dtype="f32")
    gs, cs = _summaries(w)
    G = w.group_size
    for kvh in range(2):
        for j in range(4):
            J = w.t_hist // 64 + j
            rows = ora.block_rows(w.q, 0, kvh, j, G)
            sig = ora.block_scores(rows, cs[0, kvh, :J])
            kk = w.k_cache[0, kvh].astype(np.float64)
            brute = np.array([max(float(np.mean(kk[64 * c:64 * c + 64] @ r)) for r in rows) for c in range(J)])
            assert np.max(np.abs(sig - brute)) <= 1e-5 * (1 + np.max(np.abs(brute)))
            gsig = ora.block_scores(rows, gs[0, kvh, :8 * J])
            gbrute = np.array([max(float(np.mean(kk[8 * g:8 * g + 8] @ r)) for r in rows) for g in range(8 * J)])
            assert np.max(np.abs(gsig - gbrute)) <= 1e-5 * (1 + np.max(np.abs(gbrute)))


def _brute_topk(scores, ids, k):
    """The unique k-subset whose members all beat all non-members under
    (score desc, id asc), found by enumerating every subset."""
    k = min(k, len(ids))
    found = []
    for sub in itertools.combinations(range(len(ids)), k):
        inside = set(sub)
        ok = all((scores[x] > scores[y]) or (scores[x] == scores[y] and ids[x] < ids[y])
                 for x in inside for y in range(len(ids)) if y not in inside)
        if ok:
            found.append(sorted(ids[x] for x in sub))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(12))
def test_select_topk_matches_exhaustive_enumeration(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    k = int(rng.integers(0, 5))
    # quantised scores so that ties happen often
    scores = rng.integers(-3, 4, size=n).astype(np.float32) * np.float32(0.5)
    ids = sorted(rng.choice(100, size=n, replace=False).tolist())
    assert ora.select_topk(scores, ids, k) == _brute_topk(scores, ids, k)


def test_route_unit_matches_exhaustive_scoring_on_tiny_layer():
    # the 1,024-token fp32 layer (one head, head_dim 64, top-4 chunks then top-8 groups)
    w = hi.tiny_f32()
    gs, cs = _summaries(w)
    cidx, gidx, _ = ora.route(w.q, cs, gs, w.t_hist, w.seg_len, w.top_chunks, w.top_groups, 1)
    for j in range(w.seg_len // 64):
        rows = ora.block_rows(w.q, 0, 0, j, 1)
        J = j
        full = np.array([max(float(r @ cs[0, 0, c].astype(np.float64)) for r in rows) for c in range(J)],
                        np.float64).astype(np.float32)
        # exhaustive: sort every candidate chunk
        order = sorted(range(J), key=lambda c: (-full[c], c))[:4]
        want_c = sorted(order)
        got_c = [int(x) for x in cidx[0, 0, j] if x >= 0]
        assert got_c == want_c
        assert all(x == -1 for x in cidx[0, 0, j][len(want_c):])
        cand = [8 * c + u for c in want_c for u in range(8)]
        gsc = np.array([max(float(r @ gs[0, 0, g].astype(np.float64)) for r in rows) for g in cand],
                       np.float64).astype(np.float32)
        want_g = sorted(cand[i] for i in sorted(range(len(cand)), key=lambda i: (-gsc[i], cand[i]))[:8])
        got_g = [int(x) for x in gidx[0, 0, j] if x >= 0]
        assert got_g == want_g
        # every selected group lies in a selected chunk, every selected chunk precedes block j
        assert all(g // 8 in want_c for g in got_g)
        assert all(c < J for c in got_c)


def test_route_brute_force_subsets_small_budget():
    w = hi.random_layer(seed=9, batch=1, n_q_heads=2, n_kv_heads=1, head_dim=16, t_hist=256,
                        seg_len=192, top_chunks=3, top_groups=5, dtype="bf16")
    gs, cs = _summaries(w)
    for j in range(3):
        c_sel, g_sel, sig, gids, tau = ora.route_unit(w.q, cs, gs, w.t_hist, 0, 0, j, 3, 5, 2)
        assert c_sel == _brute_topk(sig, list(range(len(sig))), 3)
        assert g_sel == _brute_topk(tau, gids, 5)


def test_fewer_candidates_than_budget_and_empty_history():
    w = hi.random_layer(seed=3, batch=1, n_q_heads=1, n_kv_heads=1, head_dim=16, t_hist=0,
                        seg_len=256, top_chunks=5, top_groups=100, dtype="bf16")
    gs, cs = _summaries(w)
    cidx, gidx, _ = ora.route(w.q, cs, gs, 0, 256, 5, 100, 1)
    assert np.all(cidx[0, 0, 0] == -1) and np.all(gidx[0, 0, 0] == -1)        # J = 0
    assert cidx[0, 0, 1].tolist() == [0, -1, -1, -1, -1]
    assert gidx[0, 0, 1, :8].tolist() == list(range(8)) and np.all(gidx[0, 0, 1, 8:] == -1)
    assert cidx[0, 0, 3, :3].tolist() == [0, 1, 2]
    assert gidx[0, 0, 3, :24].tolist() == list(range(24))


def test_selection_acceptance_rule():
    ids = [0, 1, 2, 3]
    s = np.array([1.0, 2.0, 2.0 + 1e-7, -1.0], np.float32)
    ok, ex = ora.selection_accepted([1, 2], ids, s, 2)
    assert ok and ex == 0
    ok, ex = ora.selection_accepted([0, 2], ids, s, 2)
    assert not ok
    s2 = np.array([2.0, 2.0 + 1e-6, 0.0, 0.0], np.float32)
    ok, ex = ora.selection_accepted([0], ids, s2, 1)      # near-tie exemption
    assert ok and ex == 1
    ok, _ = ora.selection_accepted([1, 1], ids, s, 2)     # duplicates rejected
    assert not ok


def test_planted_chunks_are_recalled():
    # a reduced planted workload: 1 sequence of 8,192 tokens, head layout 8/2/64
    w = hi.planted_batch(batch=1, t_total=8192, seg_len=512, n_q_heads=8, n_kv_heads=2,
                         head_dim=64, seed=55)
    gs, cs = _summaries(w)
    cidx, gidx, _ = ora.route(w.q, cs, gs, w.t_hist, w.seg_len, 16, 64, w.group_size)
    planted = set(int(c) for c in w.extra["planted_chunks"][0])
    for kvh in range(2):
        for j in range(w.seg_len // 64):
            assert planted <= set(int(c) for c in cidx[0, kvh, j])
            pg = {8 * c + u for c in planted for u in range(8)}
            assert pg <= set(int(g) for g in gidx[0, kvh, j])


def test_planted_chunks_outrank_decoys():
    """Direction control for the planted workload: 4 further chunks whose keys point
    away from the queries' planted direction (cosine -0.9) have summaries as large
    as the planted ones.  The block score is a maximum over 256 rows, so a decoy can
    come close when one row happens to point far enough away from the direction;
    on this input every planted chunk still ranks above every decoy in every block
    (a router scoring |q.S|, or the summary norm, would not), and every planted
    chunk is recalled."""
    w = hi.planted_batch(batch=1, t_total=8192, seg_len=512, n_q_heads=8, n_kv_heads=2,
                         head_dim=64, seed=55, n_decoys=4)
    gs, cs = _summaries(w)
    planted = [int(c) for c in w.extra["planted_chunks"][0]]
    decoys = [int(c) for c in w.extra["decoy_chunks"][0]]
    assert len(decoys) == 4 and not set(planted) & set(decoys)
    # the decoys' summaries are as large as the planted ones
    norm = lambda c: float(np.linalg.norm(cs[0, 0, c]))                 # noqa: E731
    assert min(norm(c) for c in decoys) > 0.8 * max(norm(c) for c in planted)
    margin = np.inf
    for kvh in range(2):
        for j in range(w.seg_len // 64):
            c_sel, _, sig, _, _ = ora.route_unit(w.q, cs, gs, w.t_hist, 0, kvh, j, 16, 64, w.group_size)
            assert set(planted) <= set(c_sel)
            margin = min(margin, min(sig[c] for c in planted) - max(sig[c] for c in decoys))
    assert margin > 0, margin
    print(f"planted chunks outrank decoys by at least {margin:.2f} in every block")


# ---------------------------------------------------------------------------
# Strictly causal routing (R-causal): a block is routed by the query block before it.
# ---------------------------------------------------------------------------

def _causal_layer(seed=21, t_hist=256, seg_len=256, dtype="f32", kc=2, kg=6):
    w = hi.random_layer(seed=seed, batch=1, n_q_heads=4, n_kv_heads=2, head_dim=32, t_hist=t_hist,
                        seg_len=seg_len, top_chunks=kc, top_groups=kg, dtype=dtype)
    q_prev = hi.prev_query_block(seed=seed, batch=1, n_q_heads=4, head_dim=32, dtype=dtype)
    return w, q_prev


def test_causal_route_scores_use_the_previous_block_rows():
    """Chunk and group scores of block j equal the mean raw logit of the rows of the
    block before it (q_prev for the first block) against each candidate's tokens,
    computed from the keys without forming a summary; the selections equal the
    exhaustive k-subset answer on those scores."""
    w, q_prev = _causal_layer()
    gs, cs = _summaries(w)
    q_all = np.concatenate([q_prev, w.q], axis=2)      # block j of the segment routes with q_all block j
    kk = w.k_cache.astype(np.float64)
    for kvh in range(2):
        for j in range(4):
            J = w.t_hist // 64 + j
            c_sel, g_sel, sig, gids, tau = ora.route_unit_causal(w.q, q_prev, cs, gs, w.t_hist, 0, kvh, j,
                                                                 w.top_chunks, w.top_groups, 2)
            rows = q_all[0, 2 * kvh:2 * kvh + 2, 64 * j:64 * j + 64].reshape(-1, 32).astype(np.float64)
            brute = np.array([max(float(np.mean(kk[0, kvh, 64 * c:64 * c + 64] @ r)) for r in rows)
                              for c in range(J)])
            assert np.max(np.abs(sig - brute)) <= 1e-5 * (1 + np.max(np.abs(brute)))
            assert c_sel == _brute_topk(sig, list(range(J)), w.top_chunks)
            gbrute = np.array([max(float(np.mean(kk[0, kvh, 8 * g:8 * g + 8] @ r)) for r in rows) for g in gids])
            assert np.max(np.abs(tau - gbrute)) <= 1e-5 * (1 + np.max(np.abs(gbrute)))
            assert g_sel == _brute_topk(tau, gids, w.top_groups)


def test_causal_route_is_blind_to_the_block_and_everything_after_it():
    """Replacing every query at or after block j's first position and every key at
    or after it leaves block j's causal selection unchanged; replacing the rows of
    the block before it does change selections (the decision really reads them)."""
    w, q_prev = _causal_layer(seed=22)
    gs, cs = _summaries(w)
    base_c, base_g, _ = ora.route_causal(w.q, q_prev, cs, gs, w.t_hist, w.seg_len, w.top_chunks, w.top_groups, 2)
    rng = np.random.default_rng(5)
    moved = 0
    for j in range(4):
        q2 = w.q.copy()
        q2[:, :, 64 * j:] = rng.standard_normal(q2[:, :, 64 * j:].shape).astype(np.float32) * 3
        w2 = hi.random_layer(seed=22, batch=1, n_q_heads=4, n_kv_heads=2, head_dim=32, t_hist=w.t_hist,
                             seg_len=w.seg_len, top_chunks=2, top_groups=6, dtype="f32")
        w2.k_cache[:, :, w.t_hist + 64 * j:] = rng.standard_normal(
            w2.k_cache[:, :, w.t_hist + 64 * j:].shape).astype(np.float32) * 3
        gs2, cs2 = _summaries(w2)
        c2, g2, _ = ora.route_causal(q2, q_prev, cs2, gs2, w.t_hist, w.seg_len, 2, 6, 2)
        np.testing.assert_array_equal(c2[:, :, j], base_c[:, :, j])
        np.testing.assert_array_equal(g2[:, :, j], base_g[:, :, j])
        # the rows that do route block j: the block before it
        q3, qp3 = w.q.copy(), q_prev.copy()
        if j > 0:
            q3[:, :, 64 * (j - 1):64 * j] = rng.standard_normal((1, 4, 64, 32)).astype(np.float32) * 3
        else:
            qp3 = rng.standard_normal(q_prev.shape).astype(np.float32) * 3
        c3, g3, _ = ora.route_causal(q3, qp3, cs, gs, w.t_hist, w.seg_len, 2, 6, 2)
        moved += int(not np.array_equal(g3[:, :, j], base_g[:, :, j]))
    assert moved >= 2


def test_causal_route_is_segmentation_invariant():
    """One 512-token segment with no history, or the same tokens as two 256-token
    segments where the second gets the first one's last query block: identical
    selections.  The first block of the sequence selects nothing."""
    w, _ = _causal_layer(seed=23, t_hist=0, seg_len=512)
    gs, cs = _summaries(w)
    c_one, g_one, _ = ora.route_causal(w.q, None, cs, gs, 0, 512, 2, 6, 2)
    c_a, g_a, _ = ora.route_causal(w.q[:, :, :256], None, cs, gs, 0, 256, 2, 6, 2)
    c_b, g_b, _ = ora.route_causal(w.q[:, :, 256:], w.q[:, :, 192:256], cs, gs, 256, 256, 2, 6, 2)
    np.testing.assert_array_equal(np.concatenate([c_a, c_b], axis=2), c_one)
    np.testing.assert_array_equal(np.concatenate([g_a, g_b], axis=2), g_one)
    assert np.all(c_one[:, :, 0] == -1) and np.all(g_one[:, :, 0] == -1)
    assert np.all(c_one[:, :, 1, 0] == 0) and np.all(c_one[:, :, 1, 1] == -1)   # only chunk 0 exists


def _layer_out(w, q, k, v, q_prev, causal):
    """Summaries, routing (block or causal) and forward of a one-sequence layer."""
    B, H, T, d = k.shape
    gs = np.zeros((B, H, T // 8, d), np.float32)
    cs = np.zeros((B, H, T // 64, d), np.float32)
    ora.build_summaries(k, 0, w.t_hist + w.seg_len, w.dtype, gs, cs)
    if causal:
        _, gidx, _ = ora.route_causal(q, q_prev, cs, gs, w.t_hist, w.seg_len, w.top_chunks, w.top_groups, 2)
    else:
        _, gidx, _ = ora.route(q, cs, gs, w.t_hist, w.seg_len, w.top_chunks, w.top_groups, 2)
    return ora.attend_fwd(q, k, v, w.t_hist, gidx, w.softmax_scale, 2)[0]


def test_causal_routing_removes_the_in_block_leak():
    """The leak: under block routing, later queries of a block can change which
    groups its earlier rows attend, so an earlier output depends on a later token.
    Steering the rows after position p of block 2 toward an unselected chunk's
    summary changes outputs at positions <= p under block routing, and changes
    nothing at positions <= p under causal routing."""
    w, q_prev = _causal_layer(seed=24, kc=1, kg=3)
    gs, cs = _summaries(w)
    j, p = 2, 10                                       # row positions 64j .. 64j+p stay fixed
    c_blk, _, _ = ora.route(w.q, cs, gs, w.t_hist, w.seg_len, 1, 3, 2)
    q2 = w.q.copy()
    for kvh in range(2):
        J = w.t_hist // 64 + j
        target = next(c for c in range(J) if c not in set(c_blk[0, kvh, j].tolist()))
        q2[0, 2 * kvh:2 * kvh + 2, 64 * j + p + 1:64 * j + 64] = 50.0 * cs[0, kvh, target]
    lo = 64 * j + p + 1
    o_blk = _layer_out(w, w.q, w.k_cache, w.v_cache, q_prev, False)
    o_blk2 = _layer_out(w, q2, w.k_cache, w.v_cache, q_prev, False)
    assert np.max(np.abs(o_blk2[:, :, 64 * j:lo] - o_blk[:, :, 64 * j:lo])) > 1e-3     # leak present
    o_c = _layer_out(w, w.q, w.k_cache, w.v_cache, q_prev, True)
    o_c2 = _layer_out(w, q2, w.k_cache, w.v_cache, q_prev, True)
    np.testing.assert_array_equal(o_c2[:, :, :lo], o_c[:, :, :lo])                     # and gone
