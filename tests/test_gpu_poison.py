"""Nothing past the live tokens is read: a layer step (hga_forward, hga_attend_bwd)
on a cache whose unused tail (K, V and the summary rows after the active segment)
holds NaN gives the same selections, outputs and gradients, bit for bit, as the
step on the same cache with a zero tail.  A read of a poisoned row would carry NaN
into a score or a gradient (a masked score still multiplies its value row)."""
import pytest
import torch

import hga_inputs as hi

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_g4_d128_b2": dict(seed=31, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, t_hist=1088, seg_len=512,
                            t_cap=1088 + 512 + 1024, top_chunks=5, top_groups=27, chunk_mean_var=0.5),
    "bf16_g8_d64_hist0": dict(seed=32, batch=1, n_q_heads=8, n_kv_heads=1, head_dim=64, t_hist=0, seg_len=256,
                              t_cap=256 + 192, top_chunks=2, top_groups=9),
    "f32_g1_d64": dict(seed=33, batch=1, n_q_heads=2, n_kv_heads=2, head_dim=64, t_hist=320, seg_len=256,
                       t_cap=320 + 256 + 640, top_chunks=3, top_groups=11, dtype="f32"),
}


@pytest.fixture(scope="module")
def chk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    from tests import hga_check
    import sparse_long_context_hga_amd as hga
    hga.lib()
    return hga_check


def _step(chk, w, poison):
    L = chk.DeviceLayer(w)
    t = w.t_hist + w.seg_len
    if poison:
        L.k[:, :, t:] = float("nan")
        L.v[:, :, t:] = float("nan")
    L.summaries(0, w.t_hist)
    if poison:
        # rows of the active segment are rewritten by the step; the ones after it stay NaN
        L.gsum[:, :, w.t_hist // 8:] = float("nan")
        L.csum[:, :, w.t_hist // 64:] = float("nan")
    L.forward()
    L.bwd()
    torch.cuda.synchronize()
    return L


@pytest.mark.parametrize("name", list(CASES))
def test_unused_cache_tail_is_never_read(chk, name):
    w = hi.random_layer(name=name, **CASES[name])
    print(f"case {name}: t_cap={w.t_cap}, live tokens {w.t_hist + w.seg_len}", flush=True)
    clean = _step(chk, w, poison=False)
    pois = _step(chk, w, poison=True)
    t = w.t_hist + w.seg_len
    for label in ("cidx", "gidx", "o", "lse", "dq", "dk", "dv"):
        a, b = getattr(clean, label), getattr(pois, label)
        assert not torch.isnan(a).any(), f"{label}: NaN in the clean step"
        assert torch.equal(a, b), f"{label} differs when the unused tail holds NaN"
    assert torch.equal(clean.gsum[:, :, : t // 8], pois.gsum[:, :, : t // 8])
    assert torch.equal(clean.csum[:, :, : t // 64], pois.csum[:, :, : t // 64])
    assert torch.isnan(pois.gsum[:, :, t // 8:]).all() and torch.isnan(pois.csum[:, :, t // 64:]).all()
