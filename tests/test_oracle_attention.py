"""Pins for the oracle's attention forward and backward (readings R-local,
R-scale, R-grad).

Checked against library routines on the CPU in float64:
  * torch.nn.functional.scaled_dot_product_attention with a boolean mask built
    from the key set (and, at full routing coverage, plain causal attention);
  * torch.logsumexp for the LSE;
  * torch.autograd through that masked attention with the history K/V as
    constants, and central differences;
plus closed-form invariants (constant V, convex hull, zero budget, unselected
history, the causal leak of block-level routing).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import hga_inputs as hi
from oracle import hga_oracle as ora


def _summaries(w):
    B, H, T, d = w.k_cache.shape
    gs = np.zeros((B, H, T // 8, d), np.float32)
    cs = np.zeros((B, H, T // 64, d), np.float32)
    ora.build_summaries(w.k_cache, 0, w.t_hist + w.seg_len, w.dtype, gs, cs)
    return gs, cs


def _mask(w, gidx):
    """Boolean [B, Hq, S, T] mask of the key set of every query row."""
    B, Hq, S, d = w.q.shape
    T = w.t_hist + w.seg_len
    G = w.group_size
    m = np.zeros((B, Hq, S, T), bool)
    for b in range(B):
        for kvh in range(w.n_kv_heads):
            for j in range(S // 64):
                J = w.t_hist // 64 + j
                for g in gidx[b, kvh, j]:
                    if g >= 0:
                        m[b, kvh * G:(kvh + 1) * G, 64 * j:64 * j + 64, 8 * g:8 * g + 8] = True
                for i in range(64):
                    m[b, kvh * G:(kvh + 1) * G, 64 * j + i, 64 * J:64 * J + i + 1] = True
    return m


def _torch_ref(w, gidx, want_grad=False):
    T = w.t_hist + w.seg_len
    G = w.group_size
    q = torch.tensor(w.q, dtype=torch.float64, requires_grad=want_grad)
    kh = torch.tensor(w.k_cache[:, :, :w.t_hist], dtype=torch.float64)                  # detached history
    vh = torch.tensor(w.v_cache[:, :, :w.t_hist], dtype=torch.float64)
    ka = torch.tensor(w.k_cache[:, :, w.t_hist:T], dtype=torch.float64, requires_grad=want_grad)
    va = torch.tensor(w.v_cache[:, :, w.t_hist:T], dtype=torch.float64, requires_grad=want_grad)
    k = torch.cat([kh, ka], 2).repeat_interleave(G, dim=1)
    v = torch.cat([vh, va], 2).repeat_interleave(G, dim=1)
    mask = torch.tensor(_mask(w, gidx))
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=w.softmax_scale)
    logits = (q @ k.transpose(-1, -2)) * w.softmax_scale
    lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
    return q, ka, va, o, lse


def _route(w):
    gs, cs = _summaries(w)
    return ora.route(w.q, cs, gs, w.t_hist, w.seg_len, w.top_chunks, w.top_groups, w.group_size)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_matches_masked_sdpa(dtype):
    w = hi.random_layer(seed=21, batch=2, n_q_heads=4, n_kv_heads=2, head_dim=32, t_hist=384,
                        seg_len=256, top_chunks=3, top_groups=13, dtype=dtype)
    _, gidx, _ = _route(w)
    o, lse = ora.attend_fwd(w.q, w.k_cache, w.v_cache, w.t_hist, gidx, w.softmax_scale, w.group_size)
    _, _, _, to, tl = _torch_ref(w, gidx)
    np.testing.assert_allclose(o, to.numpy(), atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(lse, tl.numpy(), atol=1e-12, rtol=1e-10)


def test_full_coverage_equals_dense_causal_attention():
    # the 1,024-token fp32 layer at budget 16 chunks / 128 groups covers every candidate
    w = hi.tiny_f32(full_coverage=True)
    cidx, gidx, _ = _route(w)
    o, lse = ora.attend_fwd(w.q, w.k_cache, w.v_cache, 0, gidx, w.softmax_scale, 1)
    q = torch.tensor(w.q, dtype=torch.float64)
    k = torch.tensor(w.k_cache[:, :, :1024], dtype=torch.float64)
    v = torch.tensor(w.v_cache[:, :, :1024], dtype=torch.float64)
    to = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.softmax_scale)
    np.testing.assert_allclose(o, to.numpy(), atol=1e-10)
    causal = torch.ones(1024, 1024, dtype=torch.bool).tril()
    tl = torch.logsumexp(((q @ k.transpose(-1, -2)) * w.softmax_scale).masked_fill(~causal, float("-inf")), -1)
    np.testing.assert_allclose(lse, tl.numpy(), atol=1e-10)


def test_zero_budget_is_block_diagonal_causal():
    w = hi.random_layer(seed=2, batch=1, n_q_heads=2, n_kv_heads=1, head_dim=16, t_hist=128,
                        seg_len=192, top_chunks=0, top_groups=0, dtype="f32")
    cidx, gidx, _ = _route(w)
    assert gidx.shape[-1] == 0
    o, _ = ora.attend_fwd(w.q, w.k_cache, w.v_cache, w.t_hist, gidx, w.softmax_scale, 2)
    for h in range(2):
        for j in range(3):
            J = 2 + j
            q = torch.tensor(w.q[0, h, 64 * j:64 * j + 64], dtype=torch.float64)[None]
            k = torch.tensor(w.k_cache[0, 0, 64 * J:64 * J + 64], dtype=torch.float64)[None]
            v = torch.tensor(w.v_cache[0, 0, 64 * J:64 * J + 64], dtype=torch.float64)[None]
            ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.softmax_scale)[0]
            np.testing.assert_allclose(o[0, h, 64 * j:64 * j + 64], ref.numpy(), atol=1e-12)


def test_invariants_constant_v_convex_hull_and_lse_bound():
    w = hi.random_layer(seed=4, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=16, t_hist=256,
                        seg_len=128, top_chunks=2, top_groups=9, dtype="bf16")
    _, gidx, _ = _route(w)
    vc = np.broadcast_to(np.arange(16, dtype=np.float32), w.v_cache.shape).copy()
    o, lse = ora.attend_fwd(w.q, w.k_cache, vc, w.t_hist, gidx, w.softmax_scale, 4)
    np.testing.assert_allclose(o, np.broadcast_to(np.arange(16.0), o.shape), atol=1e-12)
    o, lse = ora.attend_fwd(w.q, w.k_cache, w.v_cache, w.t_hist, gidx, w.softmax_scale, 4)
    for j in range(2):
        toks = np.concatenate([ora.key_tokens(gidx[0, 0, j]), np.arange(64 * (4 + j), 64 * (5 + j))])
        vals = w.v_cache[0, 0, toks]
        blk = o[0, :, 64 * j:64 * j + 64]
        assert np.all(blk <= vals.max(0) + 1e-12) and np.all(blk >= vals.min(0) - 1e-12)
        for h in range(4):
            for i in range(64):
                keys = np.concatenate([ora.key_tokens(gidx[0, 0, j]), np.arange(64 * (4 + j), 64 * (4 + j) + i + 1)])
                lg = w.softmax_scale * (w.k_cache[0, 0, keys].astype(np.float64) @ w.q[0, h, 64 * j + i])
                assert lse[0, h, 64 * j + i] >= lg.max() - 1e-12


def test_unselected_history_and_summaries_do_not_matter():
    w = hi.random_layer(seed=6, batch=1, n_q_heads=2, n_kv_heads=1, head_dim=16, t_hist=512,
                        seg_len=128, top_chunks=2, top_groups=6, dtype="bf16")
    gs, cs = _summaries(w)
    cidx, gidx, _ = ora.route(w.q, cs, gs, w.t_hist, w.seg_len, 2, 6, 2)
    o1, l1 = ora.attend_fwd(w.q, w.k_cache, w.v_cache, w.t_hist, gidx, w.softmax_scale, 2)
    used = set()
    for j in range(2):
        used |= set(ora.key_tokens(gidx[0, 0, j]).tolist())
    k2 = w.k_cache.copy()
    v2 = w.v_cache.copy()
    for t in range(w.t_hist):
        if t not in used:
            k2[0, 0, t] += 5.0
            v2[0, 0, t] -= 3.0
    o2, l2 = ora.attend_fwd(w.q, k2, v2, w.t_hist, gidx, w.softmax_scale, 2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # summaries only guide selection: a tiny perturbation that keeps the selection keeps the output
    cidx2, gidx2, _ = ora.route(w.q, cs * np.float32(1.0 + 2 ** -20), gs, w.t_hist, w.seg_len, 2, 6, 2)
    assert np.array_equal(gidx2, gidx)
    o3, _ = ora.attend_fwd(w.q, w.k_cache, w.v_cache, w.t_hist, gidx2, w.softmax_scale, 2)
    np.testing.assert_array_equal(o1, o3)


def test_block_level_routing_leaks_within_a_block_only():
    # seventnews, section on the causal leak: the block decision uses several query
    # positions, so a later position of a block can change an earlier position's output
    # (only through the selection); other blocks' outputs are never affected.
    w = hi.random_layer(seed=8, batch=1, n_q_heads=1, n_kv_heads=1, head_dim=16, t_hist=1024,
                        seg_len=192, top_chunks=1, top_groups=8, dtype="f32")
    gs, cs = _summaries(w)
    _, gidx, _ = ora.route(w.q, cs, gs, w.t_hist, w.seg_len, 1, 8, 1)
    o, _ = ora.attend_fwd(w.q, w.k_cache, w.v_cache, w.t_hist, gidx, w.softmax_scale, 1)
    j = 1
    cur = int(gidx[0, 0, j, 0]) // 8
    other = (cur + 3) % (w.t_hist // 64)
    q2 = w.q.copy()
    q2[0, 0, 64 * j + 63] = cs[0, 0, other] * 50.0          # steer the block to another chunk
    _, gidx2, _ = ora.route(q2, cs, gs, w.t_hist, w.seg_len, 1, 8, 1)
    assert int(gidx2[0, 0, j, 0]) // 8 == other
    o2, _ = ora.attend_fwd(q2, w.k_cache, w.v_cache, w.t_hist, gidx2, w.softmax_scale, 1)
    assert np.max(np.abs(o2[0, 0, 64 * j] - o[0, 0, 64 * j])) > 1e-3        # position 0 changed
    np.testing.assert_array_equal(o2[0, 0, :64 * j], o[0, 0, :64 * j])     # earlier block untouched


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_matches_autograd_with_detached_history(dtype):
    w = hi.random_layer(seed=31, batch=1, n_q_heads=4, n_kv_heads=2, head_dim=16, t_hist=256,
                        seg_len=256, top_chunks=3, top_groups=11, dtype=dtype)
    _, gidx, _ = _route(w)
    dq, dk, dv = ora.attend_bwd(w.q, w.k_cache, w.v_cache, w.d_o, w.t_hist, gidx, w.softmax_scale,
                                w.group_size)
    q, ka, va, o, _ = _torch_ref(w, gidx, want_grad=True)
    o.backward(torch.tensor(w.d_o, dtype=torch.float64))
    np.testing.assert_allclose(dq, q.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, ka.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, va.grad.numpy(), atol=1e-10)
    # per-chunk helper agrees with the full backward
    for cc in range(4):
        for kvh in range(2):
            dkc, dvc = ora.dkdv_active_chunk(w.q, w.k_cache, w.v_cache, w.d_o, w.t_hist, gidx, 0, kvh, cc,
                                             w.softmax_scale, w.group_size)
            np.testing.assert_allclose(dkc, dk[0, kvh, 64 * cc:64 * cc + 64], atol=1e-12)
            np.testing.assert_allclose(dvc, dv[0, kvh, 64 * cc:64 * cc + 64], atol=1e-12)


def test_backward_central_differences():
    w = hi.random_layer(seed=12, batch=1, n_q_heads=2, n_kv_heads=1, head_dim=8, t_hist=128,
                        seg_len=128, top_chunks=1, top_groups=5, dtype="f32")
    _, gidx, _ = _route(w)      # selection held fixed: routing is piecewise constant
    dq, dk, dv = ora.attend_bwd(w.q, w.k_cache, w.v_cache, w.d_o, w.t_hist, gidx, w.softmax_scale, 2)

    def loss(q, k, v):
        o, _ = ora.attend_fwd(q, k, v, w.t_hist, gidx, w.softmax_scale, 2)
        return float(np.sum(o * w.d_o))

    rng = np.random.default_rng(0)
    eps = 1e-4
    for _ in range(6):
        h, s, e = int(rng.integers(2)), int(rng.integers(128)), int(rng.integers(8))
        qp = w.q.astype(np.float64).copy(); qp[0, h, s, e] += eps
        qm = w.q.astype(np.float64).copy(); qm[0, h, s, e] -= eps
        num = (loss(qp, w.k_cache, w.v_cache) - loss(qm, w.k_cache, w.v_cache)) / (2 * eps)
        assert abs(num - dq[0, h, s, e]) < 1e-6
        t = w.t_hist + int(rng.integers(128))
        kp = w.k_cache.astype(np.float64).copy(); kp[0, 0, t, e] += eps
        km = w.k_cache.astype(np.float64).copy(); km[0, 0, t, e] -= eps
        num = (loss(w.q, kp, w.v_cache) - loss(w.q, km, w.v_cache)) / (2 * eps)
        assert abs(num - dk[0, 0, t - w.t_hist, e]) < 1e-6
        vp = w.v_cache.astype(np.float64).copy(); vp[0, 0, t, e] += eps
        vm = w.v_cache.astype(np.float64).copy(); vm[0, 0, t, e] -= eps
        num = (loss(w.q, w.k_cache, vp) - loss(w.q, w.k_cache, vm)) / (2 * eps)
        assert abs(num - dv[0, 0, t - w.t_hist, e]) < 1e-6
