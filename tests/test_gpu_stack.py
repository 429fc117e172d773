"""GPU test of the segment-wise truncated-backpropagation driver (HGAStack): two
HGA layers, each with its own K/V cache, over three segments -- forward, backward,
detach, next segment -- against the same stack computed by the oracle, segment by
segment, from the same seeded inputs.

The model around the attention is glue chosen for the test: layer 1 attends the
segment's seeded q, k, v (top-3 chunks / top-17 groups, real routing); layer 2
attends q2 = o1, k2 = the mean of o1 over the query heads of each KV head,
v2 = o1 of the first query head of each KV head, with a budget that covers every
earlier chunk and group (so its selection cannot flip under the bf16 rounding of
o1, and the oracle's fp64 layer 2 is comparable); the loss is sum(o2 * T) with a
seeded T.  Compared per segment: layer 1's selection (exact) and O / LSE of both
layers; the gradients of the segment's q, k, v (whole tensors and per 64-row
block / chunk).  Every earlier segment's tensors must receive no gradient from
later segments.  The same stack with the history in host memory (both routing
modes) must match the all-HBM stack bit for bit.
"""
import numpy as np
import pytest
import torch

import hga_inputs as hi
from oracle import hga_oracle as ora

pytestmark = pytest.mark.gpu

B, HKV, G, D, S, N_SEG = 1, 2, 4, 128, 256, 3
HQ = G * HKV
T = S * N_SEG
BUDGET1 = (3, 17)
BUDGET2 = (16, 128)          # >= every earlier chunk (at most 11) and all their groups
SCALE = 1.0 / np.sqrt(D)


@pytest.fixture(scope="module")
def chk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    from tests import hga_check
    import sparse_long_context_hga_amd as hga
    hga.lib()
    return hga_check


def _segment_inputs(s):
    """Seeded q, k, v of layer 1 and the loss weights T of segment s."""
    w = hi.random_layer(seed=200 + s, batch=B, n_q_heads=HQ, n_kv_heads=HKV, head_dim=D, t_hist=0, seg_len=S,
                        top_chunks=BUDGET1[0], top_groups=BUDGET1[1], chunk_mean_var=0.5)
    return w.q, w.k_cache[:, :, :S], w.v_cache[:, :, :S], w.d_o


class _Layer1:
    def qkv(self, h):
        return h

    def out(self, h, o):
        return o


class _Layer2:
    def qkv(self, o1):
        g = o1.view(B, HKV, G, S, D)
        k2 = g.float().mean(dim=2).to(o1.dtype).contiguous()
        v2 = g[:, :, 0].contiguous()
        return o1.contiguous(), k2, v2

    def out(self, h, o):
        return o


def _oracle_stack():
    """The same two layers and three segments in the oracle (fp64), with the
    gradients of every segment's layer-1 inputs (the glue's chain rule in numpy)."""
    k1 = np.zeros((B, HKV, T, D), np.float32)
    v1 = np.zeros_like(k1)
    k2 = np.zeros_like(k1)
    v2 = np.zeros_like(k1)
    res = []
    for s in range(N_SEG):
        q, k, v, tgt = _segment_inputs(s)
        t_hist = s * S
        k1[:, :, t_hist:t_hist + S] = k
        v1[:, :, t_hist:t_hist + S] = v
        gs1 = np.zeros((B, HKV, T // 8, D), np.float32)
        cs1 = np.zeros((B, HKV, T // 64, D), np.float32)
        ora.build_summaries(k1, 0, t_hist + S, "bf16", gs1, cs1)
        _, gidx1, _ = ora.route(q, cs1, gs1, t_hist, S, *BUDGET1, G)
        o1, lse1 = ora.attend_fwd(q, k1, v1, t_hist, gidx1, SCALE, G)
        # layer 2 (full coverage) on the oracle's own o1
        q2 = o1.astype(np.float32)
        grp = o1.reshape(B, HKV, G, S, D)
        k2[:, :, t_hist:t_hist + S] = grp.mean(axis=2)
        v2[:, :, t_hist:t_hist + S] = grp[:, :, 0]
        gs2 = np.zeros_like(gs1)
        cs2 = np.zeros_like(cs1)
        ora.build_summaries(k2, 0, t_hist + S, "bf16", gs2, cs2)
        _, gidx2, _ = ora.route(q2, cs2, gs2, t_hist, S, *BUDGET2, G)
        o2, lse2 = ora.attend_fwd(q2, k2, v2, t_hist, gidx2, SCALE, G)
        # backward: d loss / d o2 = T; layer 2, the glue, layer 1
        dq2, dk2, dv2 = ora.attend_bwd(q2, k2, v2, tgt, t_hist, gidx2, SCALE, G)
        do1 = dq2.copy().reshape(B, HKV, G, S, D)
        do1 += dk2[:, :, None] / G
        do1[:, :, 0] += dv2
        do1 = do1.reshape(B, HQ, S, D)
        dq1, dk1, dv1 = ora.attend_bwd(q, k1, v1, do1, t_hist, gidx1, SCALE, G)
        res.append(dict(gidx1=gidx1, o1=o1, lse1=lse1, o2=o2, lse2=lse2, dq=dq1, dk=dk1, dv=dv1))
    return res


def _rel(got, ref):
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))


def _block_max(got, ref):
    g = got.reshape(got.shape[0], got.shape[1], -1, 64, D)
    r = ref.reshape(g.shape)
    num = np.sqrt(((g - r) ** 2).sum(axis=(-2, -1)))
    den = np.maximum(np.sqrt((r ** 2).sum(axis=(-2, -1))), 1e-30)
    return float((num / den).max())


def test_two_layer_stack_over_three_segments(chk):
    from sparse_long_context_hga_amd.layer import HGAStack
    ref = _oracle_stack()
    stack = HGAStack([_Layer1(), _Layer2()], batch=B, n_kv_heads=HKV, head_dim=D, t_cap=T,
                     budgets=[BUDGET1, BUDGET2], softmax_scale=SCALE)
    leaves = []
    for s in range(N_SEG):
        q, k, v, tgt = _segment_inputs(s)
        print(f"segment {s}: history {stack.length} tokens", flush=True)
        x = tuple(chk.to_dev(a, "bf16").requires_grad_(True) for a in (q, k, v))
        t_dev = chk.to_dev(tgt, "f32")
        before = [[t.grad.detach().clone() for t in xs] for xs in leaves]
        loss, outs = stack.run_segment(x, lambda o2: (o2.float() * t_dev).sum())
        torch.cuda.synchronize()
        assert stack.length == (s + 1) * S
        # earlier segments are detached: nothing flowed back into their tensors
        for xs, b in zip(leaves, before):
            for t, g0 in zip(xs, b):
                assert torch.equal(t.grad, g0)
        leaves.append(x)
        r = ref[s]
        (o1, lse1, gidx1), (o2, lse2, _) = outs
        assert np.array_equal(gidx1.cpu().numpy(), r["gidx1"]), f"segment {s}: layer-1 selection differs"
        for name, got, want in (("O1", o1, r["o1"]), ("LSE1", lse1, r["lse1"]), ("O2", o2, r["o2"]),
                                ("LSE2", lse2, r["lse2"])):
            err = float(np.max(np.abs(chk.to_np(got) - want)))
            print(f"segment {s}: {name} max-abs {err:.3e}", flush=True)
            assert err <= chk.TOL_O["bf16"], (s, name, err)
        for name, t, want in (("dq", x[0], r["dq"]), ("dk", x[1], r["dk"]), ("dv", x[2], r["dv"])):
            got = chk.to_np(t.grad)
            e, eb = _rel(got, want), _block_max(got, want)
            print(f"segment {s}: {name} rel-L2 {e:.3e}, worst 64-row block {eb:.3e}", flush=True)
            assert e <= chk.TOL_GRAD_REL_L2 and eb <= chk.TOL_GRAD_REL_L2, (s, name, e, eb)


@pytest.mark.parametrize("causal", [False, True], ids=["block", "causal"])
def test_stack_with_host_history_equals_hbm(chk, causal):
    """The same stack with every layer's history in pinned host memory: per segment,
    both layers' outputs, LSE and selections and the gradients of the segment's
    inputs are bit-identical to the all-HBM stack, with block and with strictly
    causal routing."""
    from sparse_long_context_hga_amd.layer import HGAStack
    stacks = [HGAStack([_Layer1(), _Layer2()], batch=B, n_kv_heads=HKV, head_dim=D, t_cap=T,
                       budgets=[BUDGET1, BUDGET2], softmax_scale=SCALE, causal_routing=causal,
                       host_history=host, seg_len=S, n_q_heads=HQ) for host in (False, True)]
    for s in range(N_SEG):
        q, k, v, tgt = _segment_inputs(s)
        print(f"segment {s} ({'causal' if causal else 'block'} routing)", flush=True)
        t_dev = chk.to_dev(tgt, "f32")
        res = []
        for stack in stacks:
            x = tuple(chk.to_dev(a, "bf16").requires_grad_(True) for a in (q, k, v))
            _, outs = stack.run_segment(x, lambda o2: (o2.float() * t_dev).sum())
            res.append([t for layer in outs for t in layer] + [t.grad for t in x])
        torch.cuda.synchronize()
        names = ["o1", "lse1", "gidx1", "o2", "lse2", "gidx2", "dq", "dk", "dv"]
        for name, a, b_ in zip(names, *res):
            assert torch.equal(a, b_), f"segment {s}: {name} differs between host and HBM history"
