"""The seeded input generators (hga_inputs), on the CPU: bf16 rounding, determinism,
the moments of the draws, the cache layout, and the geometry of the planted batch
(keys of planted chunks at cosine 0.9 with the sequence's direction, decoys at
-0.9, queries shifted along it)."""
import numpy as np
import pytest
import torch

import hga_inputs as hi


def test_round_to_bf16_is_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)                      # bf16 spacing at 1.0
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 3 * 2 ** -8), 3.0e38],
                 np.float32)
    r = hi.round_to_bf16(x)
    assert r[0] == one
    assert r[1] == one                               # half-way, to the even mantissa (0)
    assert r[2] == one + 2 * ulp                     # half-way, to the even mantissa (2)
    assert r[3] == one + ulp                         # just above half-way
    assert r[4] == -(one + 2 * ulp)
    # every value agrees with torch's float32 -> bfloat16 conversion (round to nearest even)
    g = np.random.Generator(np.random.PCG64(5)).standard_normal(100000).astype(np.float32) * 37.0
    ref = torch.from_numpy(g).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(hi.round_to_bf16(g), ref)


def test_bf16_bits_needs_exact_values():
    x = hi.round_to_bf16(np.array([1.5, -2.25, 0.0], np.float32))
    bits = hi.bf16_bits(x).view(np.uint16)
    np.testing.assert_array_equal(bits, np.array([0x3FC0, 0xC010, 0x0000], np.uint16))
    with pytest.raises(ValueError):
        hi.bf16_bits(np.array([1.0 + 2 ** -12], np.float32))


def _layer(seed, **kw):
    base = dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, t_hist=1024, seg_len=512, top_chunks=4,
                top_groups=16)
    base.update(kw)
    return hi.random_layer(seed=seed, **base)


def test_layers_are_deterministic_per_seed():
    a, b, c = _layer(3), _layer(3), _layer(4)
    for f in ("q", "k_cache", "v_cache", "d_o"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
        assert not np.array_equal(getattr(a, f), getattr(c, f))
    # the streams of Q, K, V and dO are distinct
    assert not np.array_equal(a.q[:, :2], a.k_cache[:, :, :512])


def test_moments_and_cache_layout():
    w = _layer(6, t_cap=1024 + 512 + 256, chunk_mean_var=0.5, dtype="bf16")
    t = w.t_hist + w.seg_len
    for f, var in (("q", 1.0), ("v_cache", 1.0), ("k_cache", 1.5), ("d_o", 1.0)):
        x = getattr(w, f)
        if f.endswith("cache"):
            x = x[:, :, :t]
        assert abs(float(x.mean())) < 0.01, f
        assert abs(float(x.var()) / var - 1.0) < 0.02, f
        assert np.array_equal(hi.round_to_bf16(x), x), f"{f} is not bf16-exact"
    # keys carry a per-(sequence, KV head, chunk) mean of variance 0.5 (plus 1/64 of noise)
    chunk_means = w.k_cache[:, :, :t].reshape(w.batch, w.n_kv_heads, t // 64, 64, w.head_dim).mean(axis=3)
    assert abs(float(chunk_means.var()) / (0.5 + 1 / 64) - 1.0) < 0.05
    # positions past the live tokens are zero
    assert not w.k_cache[:, :, t:].any() and not w.v_cache[:, :, t:].any()


def test_planted_batch_geometry():
    w = hi.planted_batch(batch=2, t_total=4096, seg_len=512, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         n_planted=4, n_decoys=4, seed=9)
    pl, de = w.extra["planted_chunks"], w.extra["decoy_chunks"]
    n_hist = w.t_hist // 64
    for b in range(w.batch):
        both = np.concatenate([pl[b], de[b]])
        assert len(set(both.tolist())) == 8 and both.min() >= 0 and both.max() < n_hist
        assert np.all(np.diff(pl[b]) > 0) and np.all(np.diff(de[b]) > 0)

        def mean_dir(chunks):
            k = np.concatenate([w.k_cache[b, :, 64 * c:64 * c + 64] for c in chunks], axis=1).astype(np.float64)
            k /= np.linalg.norm(k, axis=-1, keepdims=True)
            return k.reshape(-1, w.head_dim).mean(axis=0)

        mp, md = mean_dir(pl[b]), mean_dir(de[b])
        # unit keys 0.9 u + 0.44 w (w orthogonal to u, random): their mean is about 0.9 u
        assert abs(np.linalg.norm(mp) - 0.9) < 0.03 and abs(np.linalg.norm(md) - 0.9) < 0.03
        cos_pd = mp @ md / (np.linalg.norm(mp) * np.linalg.norm(md))
        assert cos_pd < -0.99                          # decoys point the other way
        others = [c for c in range(n_hist) if c not in set(both.tolist())][:8]
        assert np.linalg.norm(mean_dir(others)) < 0.15  # no common direction elsewhere
        # queries: N(0, I) shifted by 1.0 along the same direction (the mean over 2,048
        # query rows keeps noise of norm about sqrt(64 / 2048) = 0.18)
        qm = w.q[b].reshape(-1, w.head_dim).astype(np.float64).mean(axis=0)
        assert abs(np.linalg.norm(qm) - 1.0) < 0.06
        assert qm @ mp / (np.linalg.norm(qm) * np.linalg.norm(mp)) > 0.95


def test_rollout_segments_and_generation_batches():
    a0, a1 = hi.rollout_segment(0, n_q_heads=2, n_kv_heads=1, head_dim=64, seg_len=128), \
        hi.rollout_segment(1, n_q_heads=2, n_kv_heads=1, head_dim=64, seg_len=128)
    b0 = hi.rollout_segment(0, n_q_heads=2, n_kv_heads=1, head_dim=64, seg_len=128)
    for x, y, z in zip(a0, b0, a1):
        np.testing.assert_array_equal(x, y)
        assert not np.array_equal(x, z)
    w = hi.decode_batch(seed=3, batch=3, n_q_heads=4, n_kv_heads=2, head_dim=64, t_cap=512, pos=[511, 10, -1],
                        top_chunks=2, top_groups=8)
    assert w.q.shape == (3, 4, 64) and w.k_cache.shape == (3, 2, 512, 64)
    assert list(w.pos) == [511, 10, -1] and w.group_size == 2
