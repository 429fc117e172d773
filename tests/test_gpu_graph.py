"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

No call records a memset or allocates, so a whole layer step (hga_forward, then
hga_attend_bwd) and a generation step that allocates nothing
(hga_decode_step_noalloc) can be captured once and replayed.  Every replay must
reproduce the eager call bit for bit; each replay follows a reset of the outputs
and is followed by an eager call of its own, with synchronizations between.
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


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(g, fn, outputs, ref, label, n=3):
    for r in range(n):
        for t in outputs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs, ref)):
            assert torch.equal(a, b), f"{label}: replay {r}, output {i} differs from the eager call"
        fn()                                    # eager work between the replays
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs, ref)):
            assert torch.equal(a, b), f"{label}: eager call after replay {r}, output {i} differs"
    print(f"{label}: {n} replays identical to the eager call", flush=True)


def test_layer_step_replays_in_a_graph(chk):
    w = hi.random_layer(seed=121, batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, t_hist=1024, seg_len=512,
                        top_chunks=4, top_groups=20, chunk_mean_var=0.5)
    L = chk.DeviceLayer(w)
    L.summaries(0, w.t_hist)

    def step():
        L.forward()
        L.bwd()

    step()
    torch.cuda.synchronize()
    outputs = [L.o, L.lse, L.dq, L.dk, L.dv, L.cidx, L.gidx]
    ref = [t.clone() for t in outputs]
    g = _capture(step)
    _replays_match(g, step, outputs, ref, "layer step")


def test_noalloc_generation_step_replays_in_a_graph(chk):
    import sparse_long_context_hga_amd as hga
    w = hi.decode_batch(seed=122, batch=4, n_q_heads=16, n_kv_heads=4, head_dim=128, t_cap=4096,
                        pos=[4095, 3000, 2047, 100], top_chunks=8, top_groups=40, chunk_mean_var=0.5)
    B, H, T, d = w.k_cache.shape
    gs_np = np.zeros((B, H, T // 8, d), np.float32)
    cs_np = np.zeros((B, H, T // 64, d), np.float32)
    ora.build_summaries(w.k_cache, 0, T, w.dtype, gs_np, cs_np)
    shape = hga.make_shape(B, w.n_q_heads, H, d, w.top_chunks, w.top_groups, "bf16", w.softmax_scale)
    q, k, v = (chk.to_dev(x, "bf16") for x in (w.q, w.k_cache, w.v_cache))
    gs, cs = chk.to_dev(gs_np, "bf16"), chk.to_dev(cs_np, "bf16")
    pos = torch.tensor(w.pos, dtype=torch.int32, device="cuda")
    cidx = torch.empty(B, H, w.top_chunks, dtype=torch.int32, device="cuda")
    gidx = torch.empty(B, H, w.top_groups, dtype=torch.int32, device="cuda")
    o = torch.empty(B, w.n_q_heads, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, w.n_q_heads, dtype=torch.float32, device="cuda")

    def step():
        hga.hga_decode_step_noalloc(shape, q, k, v, cs, gs, T, pos, cidx, gidx, o, lse)

    step()
    torch.cuda.synchronize()
    outputs = [o, lse, cidx, gidx, gs, cs]
    ref = [t.clone() for t in outputs]
    g = _capture(step)
    # the summary tables are inputs as well as outputs: a replay must find them as the
    # eager call left them, so only O, LSE and the selections are reset before it
    _replays_match(g, step, outputs[:4], ref[:4], "generation step (no allocation)")
    for a, b in zip(outputs[4:], ref[4:]):
        assert torch.equal(a, b)
