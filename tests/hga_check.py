"""Helpers that run the HIP library on seeded workloads and compare with the CPU oracle.

Used by the GPU parity tests and by the smoke check.  Every expected value comes
from the oracle; the oracle never receives anything the GPU produced.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np
import torch

import hga_inputs as hi
import sparse_long_context_hga_amd as hga
from sparse_long_context_hga_amd.layer import HGALayerBuffers
from oracle import hga_oracle as ora

# Acceptance thresholds (O / LSE max-abs per dtype, gradients relative L2, near-tie margin).
TOL_O = {"bf16": 2e-2, "f32": 1e-4}
TOL_GRAD_REL_L2 = 3e-2
NEAR_TIE_REL = 1e-5


def tdt(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(tdt(dtype)).contiguous()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def shape_of(w: hi.Workload, top_chunks: Optional[int] = None, top_groups: Optional[int] = None):
    return hga.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim,
                          w.top_chunks if top_chunks is None else top_chunks,
                          w.top_groups if top_groups is None else top_groups, w.dtype, w.softmax_scale)


class DeviceLayer(HGALayerBuffers):
    """Device copies of a workload plus the buffers of one layer step."""

    def __init__(self, w: hi.Workload, device="cuda"):
        self.w = w
        do = to_dev(w.d_o, w.dtype, device) if w.d_o is not None else None
        super().__init__(shape_of(w), to_dev(w.q, w.dtype, device), to_dev(w.k_cache, w.dtype, device),
                         to_dev(w.v_cache, w.dtype, device), w.t_hist, do)


# ---------------------------------------------------------------- oracle side
def oracle_summaries(w: hi.Workload) -> Tuple[np.ndarray, np.ndarray]:
    B, H, T, d = w.k_cache.shape
    gs = np.zeros((B, H, T // 8, d), np.float32)
    cs = np.zeros((B, H, T // 64, d), np.float32)
    ora.build_summaries(w.k_cache, 0, w.t_hist + w.seg_len, w.dtype, gs, cs)
    return gs, cs


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))


def check_route_unit(w, gs, cs, b, kvh, j, cidx_row, gidx_row, causal=False, q_prev=None) -> int:
    """Acceptance of the GPU selection of one unit against oracle scores (block
    routing, or causal routing with the previous segment's last block q_prev).
    Returns the number of near-tie exemptions; raises AssertionError on failure."""
    J = w.t_hist // 64 + j
    if causal and J == 0:
        assert all(x == -1 for x in cidx_row) and all(x == -1 for x in gidx_row)
        return 0
    rows = (ora.causal_routing_rows(w.q, q_prev, b, kvh, j, w.group_size) if causal
            else ora.block_rows(w.q, b, kvh, j, w.group_size))
    return check_selection(rows, J, gs, cs, b, kvh, cidx_row, gidx_row, w.top_chunks, w.top_groups,
                           (b, kvh, j))


def check_selection(rows, J, gs, cs, b, kvh, cidx_row, gidx_row, top_chunks, top_groups, where) -> int:
    """Acceptance of a GPU selection made by the given query rows over candidate
    chunks [0, J), against the oracle's scores.  Returns the near-tie exemptions."""
    sig = ora.block_scores(rows, cs[b, kvh, :J])
    csel = [int(x) for x in cidx_row if x >= 0]
    assert all(x == -1 for x in cidx_row[len(csel):]), "chunk list not -1 padded at the end"
    assert csel == sorted(csel), "chunk ids not ascending"
    ok, ex1 = ora.selection_accepted(csel, list(range(J)), sig, top_chunks, NEAR_TIE_REL)
    assert ok, f"chunk selection rejected at unit {where}: {csel}"
    gids = [8 * c + u for c in csel for u in range(8)]
    tau = ora.block_scores(rows, gs[b, kvh, gids]) if gids else np.zeros(0, np.float32)
    gsel = [int(x) for x in gidx_row if x >= 0]
    assert all(x == -1 for x in gidx_row[len(gsel):]), "group list not -1 padded at the end"
    assert gsel == sorted(gsel), "group ids not ascending"
    ok, ex2 = ora.selection_accepted(gsel, gids, tau, top_groups, NEAR_TIE_REL)
    assert ok, f"group selection rejected at unit {where}: {gsel}"
    return ex1 + ex2


def oracle_route(w, gs, cs):
    return ora.route(w.q, cs, gs, w.t_hist, w.seg_len, w.top_chunks, w.top_groups, w.group_size)


def fwd_errors(w, o_gpu, lse_gpu, gidx, units=None) -> Tuple[float, float]:
    """Max-abs error of O and LSE against the oracle on the given group selection."""
    G = w.group_size
    eo = el = 0.0
    if units is None:
        o, lse = ora.attend_fwd(w.q, w.k_cache, w.v_cache, w.t_hist, gidx, w.softmax_scale, G)
        return float(np.max(np.abs(o_gpu - o))), float(np.max(np.abs(lse_gpu - lse)))
    for (b, kvh, j) in units:
        ou, lu = ora.attend_fwd_unit(w.q, w.k_cache, w.v_cache, w.t_hist, gidx[b, kvh, j], b, kvh, j,
                                     w.softmax_scale, G)
        h0 = kvh * G
        og = o_gpu[b, h0:h0 + G, 64 * j:64 * j + 64].reshape(-1, w.head_dim)
        lg = lse_gpu[b, h0:h0 + G, 64 * j:64 * j + 64].reshape(-1)
        eo = max(eo, float(np.max(np.abs(og - ou))))
        el = max(el, float(np.max(np.abs(lg - lu))))
    return eo, el


def bwd_errors(w, dq_gpu, dk_gpu, dv_gpu, gidx, units=None, chunks=None) -> Dict[str, float]:
    """Relative-L2 errors of dQ, dK_active, dV_active against the oracle."""
    G = w.group_size
    if units is None:
        dq, dk, dv = ora.attend_bwd(w.q, w.k_cache, w.v_cache, w.d_o, w.t_hist, gidx, w.softmax_scale, G)
        return {"dq": rel_l2(dq_gpu, dq), "dk": rel_l2(dk_gpu, dk), "dv": rel_l2(dv_gpu, dv)}
    got, ref = [], []
    for (b, kvh, j) in units:
        r = ora.dq_unit(w.q, w.k_cache, w.v_cache, w.d_o, w.t_hist, gidx[b, kvh, j], b, kvh, j,
                        w.softmax_scale, G)
        got.append(dq_gpu[b, kvh * G:(kvh + 1) * G, 64 * j:64 * j + 64].reshape(-1, w.head_dim))
        ref.append(r)
    out = {"dq": rel_l2(np.concatenate(got), np.concatenate(ref))}
    gk, gv, rk, rv = [], [], [], []
    for (b, kvh, cc) in chunks:
        dk, dv = ora.dkdv_active_chunk(w.q, w.k_cache, w.v_cache, w.d_o, w.t_hist, gidx, b, kvh, cc,
                                       w.softmax_scale, G)
        gk.append(dk_gpu[b, kvh, 64 * cc:64 * cc + 64]); rk.append(dk)
        gv.append(dv_gpu[b, kvh, 64 * cc:64 * cc + 64]); rv.append(dv)
    out["dk"] = rel_l2(np.concatenate(gk), np.concatenate(rk))
    out["dv"] = rel_l2(np.concatenate(gv), np.concatenate(rv))
    return out


def smoke_check() -> None:
    """One small bf16 step (route + forward + backward) on cuda:0, checked against the oracle."""
    w = hi.random_layer(seed=101, batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, t_hist=512,
                        seg_len=256, top_chunks=4, top_groups=20, chunk_mean_var=0.5,
                        name="smoke_ctx768")
    print(f"smoke: {w.name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim} "
          f"t_hist={w.t_hist} S={w.seg_len}", flush=True)
    L = DeviceLayer(w)
    L.summaries(0, w.t_hist + w.seg_len)
    L.route()
    L.fwd()
    L.bwd()
    torch.cuda.synchronize()
    gs, cs = oracle_summaries(w)
    assert np.array_equal(to_np(L.gsum), gs) and np.array_equal(to_np(L.csum), cs), "summaries differ"
    cidx = L.cidx.cpu().numpy()
    gidx = L.gidx.cpu().numpy()
    _, ogidx, _ = oracle_route(w, gs, cs)
    for kvh in range(w.n_kv_heads):
        for j in range(w.seg_len // 64):
            check_route_unit(w, gs, cs, 0, kvh, j, cidx[0, kvh, j], gidx[0, kvh, j])
    # attention on the oracle's selection
    og = torch.from_numpy(ogidx).cuda()
    L.fwd(og)
    L.bwd(og)
    torch.cuda.synchronize()
    eo, el = fwd_errors(w, to_np(L.o), to_np(L.lse), ogidx)
    errs = bwd_errors(w, to_np(L.dq), to_np(L.dk), to_np(L.dv), ogidx)
    print(f"smoke: O max-abs {eo:.3e} LSE max-abs {el:.3e} grads rel-L2 {errs}", flush=True)
    assert eo <= TOL_O["bf16"] and el <= TOL_O["bf16"]
    assert all(v <= TOL_GRAD_REL_L2 for v in errs.values())
    print("smoke: ok", flush=True)
