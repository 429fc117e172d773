"""GPU tests of the host-RAM history tier (hga_stage_history, HGAHostKVCache): the
detached history's K/V in pinned host memory, the summary tables in HBM, and per
segment a staging cache in HBM holding only the selected history groups.

  * the staging call itself: the renumbered selection and the staged rows are
    exactly what the documented mapping gives (slot s = the s-th distinct selected
    history group, active ids after the staging area), on a history longer than
    the staging area;
  * the autograd op over consecutive segments with a host-tier cache gives, bit
    for bit, the outputs, selections and gradients of the same op with the whole
    history in HBM (whose parity with the oracle the other tests establish): one
    case whose staging area holds the whole history, one where it is far smaller,
    each with block and with strictly causal routing.
"""
import numpy as np
import pytest
import torch

import hga_inputs as hi

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hga():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import sparse_long_context_hga_amd as hga
    hga.lib()
    return hga


def _expected_stage(gidx, t_hist, stage_hist):
    """Reference renumbering and slot lists, from the definition (numpy)."""
    B, H = gidx.shape[:2]
    out = np.full_like(gidx, -1)
    slots = {}
    for b in range(B):
        for h in range(H):
            ids = gidx[b, h].ravel()
            hist = sorted(set(int(x) for x in ids if 0 <= x < t_hist // 8))
            pos = {g: s for s, g in enumerate(hist)}
            m = [(-1 if x < 0 else pos[int(x)] if x < t_hist // 8 else stage_hist // 8 + int(x) - t_hist // 8)
                 for x in ids]
            out[b, h] = np.asarray(m, np.int32).reshape(gidx.shape[2:])
            slots[(b, h)] = hist
    return out, slots


def test_stage_history_mapping_and_rows(hga):
    """Route a segment over 3,840 history tokens (budget 4 chunks / 12 groups, 4
    blocks: at most 48 groups = 384 tokens staged), stage, and check every index and
    every staged row."""
    w = hi.random_layer(seed=301, batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128, t_hist=3840, seg_len=256,
                        top_chunks=4, top_groups=12, chunk_mean_var=0.5, backward=False)
    shape = hga.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.top_chunks, w.top_groups, "bf16",
                           w.softmax_scale)
    dt = torch.bfloat16
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dt).contiguous()   # noqa: E731
    k, v = dev(w.k_cache), dev(w.v_cache)
    T = w.t_hist + w.seg_len
    gs = torch.zeros(w.batch, w.n_kv_heads, T // 8, w.head_dim, dtype=dt, device="cuda")
    cs = torch.zeros(w.batch, w.n_kv_heads, T // 64, w.head_dim, dtype=dt, device="cuda")
    nb = w.seg_len // 64
    cidx = torch.empty(w.batch, w.n_kv_heads, nb, w.top_chunks, dtype=torch.int32, device="cuda")
    gidx = torch.empty(w.batch, w.n_kv_heads, nb, w.top_groups, dtype=torch.int32, device="cuda")
    hga.hga_build_summaries(shape, k, T, 0, T, gs, cs)
    hga.hga_route(shape, dev(w.q), cs, gs, T, w.t_hist, w.seg_len, cidx, gidx)
    k_host = k.cpu().pin_memory()
    v_host = v.cpu().pin_memory()
    stage_hist = hga.hga_stage_history_min(shape, w.t_hist, w.seg_len)
    assert stage_hist == 384
    stage_cap = stage_hist + w.seg_len
    k_st = torch.full((w.batch, w.n_kv_heads, stage_cap, w.head_dim), 7.0, dtype=dt, device="cuda")
    v_st = torch.full_like(k_st, 7.0)
    gst = torch.empty_like(gidx)
    hga.hga_stage_history(shape, k_host, v_host, T, w.t_hist, w.seg_len, gidx, k_st, v_st, stage_cap, stage_hist,
                          gst)
    torch.cuda.synchronize()
    g = gidx.cpu().numpy()
    want, slots = _expected_stage(g, w.t_hist, stage_hist)
    np.testing.assert_array_equal(gst.cpu().numpy(), want)
    ks, vs = k_st.cpu(), v_st.cpu()
    kh, vh = k_host, v_host
    n_staged = 0
    for (b, h), hist in slots.items():
        for s, grp in enumerate(hist):
            assert torch.equal(ks[b, h, 8 * s:8 * s + 8], kh[b, h, 8 * grp:8 * grp + 8])
            assert torch.equal(vs[b, h, 8 * s:8 * s + 8], vh[b, h, 8 * grp:8 * grp + 8])
        # rows of unused slots are untouched
        assert torch.all(ks[b, h, 8 * len(hist):stage_hist] == 7.0)
        n_staged += len(hist)
    print(f"staged {n_staged} history groups for {len(slots)} (sequence, KV head) pairs", flush=True)


def test_stage_history_at_the_maximum_history(hga):
    """Staging at the library's largest cache (8,192 chunks: 524,160 history tokens,
    65,520 history groups, every word of the selection bitmap in use): route two
    blocks over all 8,190-8,191 earlier chunks, stage, and check every index and row."""
    B, Hq, Hkv, d, S = 1, 2, 1, 64, 128
    T = 64 * 8192
    th = T - S
    rng = np.random.default_rng(77)
    kc = hi.round_to_bf16(rng.standard_normal((B, Hkv, T, d), dtype=np.float32))
    vc = hi.round_to_bf16(rng.standard_normal((B, Hkv, T, d), dtype=np.float32))
    q = hi.round_to_bf16(rng.standard_normal((B, Hq, S, d), dtype=np.float32))
    shape = hga.make_shape(B, Hq, Hkv, d, 16, 64, "bf16")
    dt = torch.bfloat16
    k = torch.from_numpy(kc).to("cuda").to(dt).contiguous()
    gs = torch.zeros(B, Hkv, T // 8, d, dtype=dt, device="cuda")
    cs = torch.zeros(B, Hkv, T // 64, d, dtype=dt, device="cuda")
    hga.hga_build_summaries(shape, k, T, 0, T, gs, cs)
    cidx = torch.empty(B, Hkv, S // 64, 16, dtype=torch.int32, device="cuda")
    gidx = torch.empty(B, Hkv, S // 64, 64, dtype=torch.int32, device="cuda")
    hga.hga_route(shape, torch.from_numpy(q).to("cuda").to(dt).contiguous(), cs, gs, T, th, S, cidx, gidx)
    del k
    k_host = torch.from_numpy(kc).to(dt).pin_memory()
    v_host = torch.from_numpy(vc).to(dt).pin_memory()
    sh = hga.hga_stage_history_min(shape, th, S)
    cap = sh + S
    k_st = torch.full((B, Hkv, cap, d), 7.0, dtype=dt, device="cuda")
    v_st = torch.full_like(k_st, 7.0)
    gst = torch.empty_like(gidx)
    hga.hga_stage_history(shape, k_host, v_host, T, th, S, gidx, k_st, v_st, cap, sh, gst)
    torch.cuda.synchronize()
    g = gidx.cpu().numpy()
    assert g.max() >= 8 * 4096, "the selection should reach the second half of the history"
    want, slots = _expected_stage(g, th, sh)
    np.testing.assert_array_equal(gst.cpu().numpy(), want)
    ks, vs = k_st.cpu(), v_st.cpu()
    hist = slots[(0, 0)]
    for s_, grp in enumerate(hist):
        assert torch.equal(ks[0, 0, 8 * s_:8 * s_ + 8], k_host[0, 0, 8 * grp:8 * grp + 8])
        assert torch.equal(vs[0, 0, 8 * s_:8 * s_ + 8], v_host[0, 0, 8 * grp:8 * grp + 8])
    assert torch.all(ks[0, 0, 8 * len(hist):sh] == 7.0)
    print(f"staged {len(hist)} of {th // 8} history groups, highest id {max(hist)}", flush=True)


CASES = {
    # the staging area holds the whole history (512 tokens)
    "g4_d128_s256": dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, seg_len=256, n_seg=3,
                         top_chunks=3, top_groups=17),
    # 7 segments of history (896 tokens) through a staging area of 128 tokens
    "g2_d64_s128_small_stage": dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, seg_len=128, n_seg=8,
                                    top_chunks=2, top_groups=8),
}


@pytest.mark.parametrize("causal", [False, True], ids=["block", "causal"])
@pytest.mark.parametrize("name", list(CASES))
def test_host_tier_equals_hbm_history(hga, name, causal):
    """Every segment's outputs, selection and gradients are bit-identical with the
    history in host memory and in HBM, with block and with strictly causal routing."""
    from sparse_long_context_hga_amd.layer import HGAHostKVCache, HGAKVCache, hga_attention
    c = CASES[name]
    B, Hq, Hkv, d, S, n_seg = c["batch"], c["n_q_heads"], c["n_kv_heads"], c["head_dim"], c["seg_len"], c["n_seg"]
    kc, kg = c["top_chunks"], c["top_groups"]
    T = S * n_seg
    dev_cache = HGAKVCache(B, Hkv, d, T, torch.bfloat16)
    host_cache = HGAHostKVCache(B, Hkv, d, T, S, Hq, kc, kg, torch.bfloat16)
    print(f"case {name} ({'causal' if causal else 'block'} routing): staging area {host_cache.stage_hist} tokens "
          f"for up to {T - S} history tokens", flush=True)
    for s in range(n_seg):
        w = hi.random_layer(seed=400 + s, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, t_hist=0, seg_len=S,
                            top_chunks=kc, top_groups=kg, chunk_mean_var=0.5)
        res = []
        for cache in (dev_cache, host_cache):
            xs = [torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16).requires_grad_(True)
                  for a in (w.q, w.k_cache[:, :, :S], w.v_cache[:, :, :S])]
            o, lse, gidx = hga_attention(*xs, cache, kc, kg, causal_routing=causal)
            (o.float() * torch.from_numpy(w.d_o).cuda()).sum().backward()
            cache.commit(S)
            res.append([o.detach(), lse, gidx] + [x.grad for x in xs])
        torch.cuda.synchronize()
        for label, a, b_ in zip(("o", "lse", "group_idx", "dq", "dk", "dv"), *res):
            assert torch.equal(a, b_), f"{name}, segment {s}: {label} differs between the tiers"
    print(f"case {name}: {n_seg} segments bit-identical", flush=True)


def test_host_tier_rejects_a_larger_budget(hga):
    """The staging area is sized for the cache's budget: a call with more groups per
    block is refused before anything is written or launched."""
    from sparse_long_context_hga_amd.layer import HGAHostKVCache, hga_attention
    cache = HGAHostKVCache(1, 2, 64, 512, 128, 4, 2, 8, torch.bfloat16)
    q = torch.zeros(1, 4, 128, 64, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="sized for"):
        hga_attention(q, kv, kv, cache, 2, 16)
    assert cache.length == 0

