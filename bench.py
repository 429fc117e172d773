#!/usr/bin/env python3
"""Throughput of the HGA routed-attention layer step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
build the active segment's summaries, route every query block, attention
forward, attention backward (dQ and the active segment's dK/dV).  Inputs are
resident in HBM before the timed region; the history summaries are built once,
untimed, like a cache that earlier segments filled.

Default workload: a Qwen3-8B-shaped attention layer (32 query / 8 KV heads,
head_dim 128, bf16) at 16,384 tokens of context: 14,336 detached history tokens
plus a 2,048-token active segment, top-16 chunks / top-64 groups, block-structured
keys.  Prints one JSON line (tokens/s of the active segment, whole job).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--routing block|causal]
                    [--no-cpu-baseline]

--routing causal times the strictly causal variant (each block routed by the
block before it, hga_route_causal); the default is block routing.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "HGA attention-layer tokens/s (fwd+bwd) at 16K ctx; % of HBM and MFMA roofline"


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=300,
                   help="untimed steps first (default 300): the GPU clock ramps up over the first tens of "
                        "milliseconds of sustained work, so the timed steps see its steady state")
    p.add_argument("--workload", default="qwen3_8b_layer_ctx16k",
                   choices=["qwen3_8b_layer_ctx16k", "qwen3_8b_layer_ctx4k", "planted_b8_ctx32k",
                            "decode_b8_ctx32k", "decode_b64_ctx16k", "rollout_131k"],
                   help="decode_b8_ctx32k / decode_b64_ctx16k time the generation path (hga_decode_route + "
                        "hga_decode_attend) for 8 sequences at 32K / 64 at 16K; "
                        "rollout_131k the 64-segment forward rollout")
    p.add_argument("--history", default="hbm", choices=["hbm", "host"],
                   help="hbm: the detached history is resident in HBM; host: in pinned host memory, with the "
                        "selected groups staged into HBM after routing (hga_stage_history); the step rate then "
                        "includes the host link")
    p.add_argument("--routing", default="block", choices=["block", "causal"],
                   help="block: each block routes itself (hga_route); causal: the block before it routes it")
    p.add_argument("--marked-steps", type=int, default=20,
                   help="steps run after the timed region with every kernel timed from its own dispatch "
                        "(HIP events recorded by the launches; default 20)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    p.add_argument("--cold", action="store_true",
                   help="write 512 MiB between timed steps (outside the timing) so that no step finds its "
                        "inputs in the 256 MB MALL; the step time is then the sum of per-step HIP events")
    p.add_argument("--no-calibration", action="store_true",
                   help="skip the measurement of the box's achievable copy bandwidth and bf16 GEMM rate")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="first run a fill and a scale-copy kernel of this size (reference for HBM counters)")
    p.add_argument("--mfma-summary", metavar="COUNTER_CSV",
                   help="no GPU work: reduce a rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 counter_collection.csv "
                        "into the MFMA summary under profiles/")
    p.add_argument("--stall-summary", nargs="+", metavar="COUNTER_CSV",
                   help="no GPU work: reduce rocprofv3 --pmc counter_collection.csv files of SQ wave counters "
                        "(SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_*, ...) into the "
                        "wave-state summary under profiles/")
    p.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU work: reduce two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                        "WRITE_SIZE) of a --copy-calibration-mib run into the traffic summary under profiles/")
    return p.parse_args()


# ------------------------------------------------------------------ algorithmic work
def algorithmic_work(w, gidx):
    """Algorithmic HBM bytes and MFMA flops per kernel for one step, from the
    selection actually made (number of valid groups per unit)."""
    import numpy as np
    B, Hq, Hkv, d, S, G = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seg_len, w.group_size
    el = 2 if w.dtype == "bf16" else 4
    nb = S // 64
    R = G * 64                                       # query rows per unit
    n_sel = (gidx >= 0).sum(axis=-1) * 8             # selected tokens per unit [B,Hkv,nb]
    tok_sel = float(n_sel.sum())
    units = B * Hkv * nb
    loc_keys = 32.5                                  # causal own-chunk keys per row (mean)
    kv_sel = tok_sel * d * el * 2                    # gathered K and V
    kv_loc = units * 64 * d * el * 2
    q_bytes = B * Hq * S * d * el
    # forward: Q, gathered K/V, own chunk K/V, O, LSE, selection
    fwd_bytes = q_bytes + kv_sel + kv_loc + q_bytes + B * Hq * S * 4 + gidx.size * 4
    fwd_flops = 2 * 2 * R * d * tok_sel + 2 * 2 * R * d * loc_keys * units
    # dQ: Q, dO, O, LSE, gathered K/V, own chunk K/V, dQ, D
    dq_bytes = 3 * q_bytes + kv_sel + kv_loc + q_bytes + 2 * B * Hq * S * 4 + gidx.size * 4
    dq_flops = 3 * 2 * R * d * tok_sel + 3 * 2 * R * d * loc_keys * units
    # dK/dV: own K/V, Q/dO rows of every visiting block, dK, dV
    act_lo = w.t_hist // 8
    visits = 0
    sel_act_tokens = 0
    for b in range(B):
        for h in range(Hkv):
            for j in range(nb):
                g = gidx[b, h, j]
                g = g[g >= act_lo]
                sel_act_tokens += 8 * len(g)
                visits += len(np.unique(g // 8))
    visits += units                                   # own block of every chunk
    dkdv_bytes = kv_loc + visits * 2 * R * d * el + visits * 2 * R * 4 + kv_loc
    dkdv_flops = 4 * 2 * R * d * (sel_act_tokens + loc_keys * units)
    # routing: Q block rows x candidate chunk summaries, then 8*k_c group summaries
    J = np.arange(nb) + w.t_hist // 64
    route_flops = B * Hkv * float(np.sum(2 * R * d * (J + 8 * np.minimum(w.top_chunks, J))))
    route_bytes = q_bytes + B * Hkv * (w.t_hist + S) // 64 * d * el + gidx.size * 4 * 2
    sum_bytes = B * Hkv * S * d * el + B * Hkv * (S // 8 + S // 64) * d * el
    return {
        "summaries": {"bytes": sum_bytes, "flops": 0.0},
        "route": {"bytes": route_bytes, "flops": route_flops},
        "attend_fwd": {"bytes": fwd_bytes, "flops": fwd_flops, "gather_bytes": kv_sel},
        # routing and attention in one work-group per unit: Q is read once for both
        # the same with strictly causal routing: the routing rows are the block before
        # (read once more), the attention reads the block's own rows
        "route_attend_causal": {"bytes": route_bytes + fwd_bytes, "flops": route_flops + fwd_flops,
                                "gather_bytes": kv_sel},
        "route_attend": {"bytes": route_bytes + fwd_bytes - q_bytes, "flops": route_flops + fwd_flops,
                         "gather_bytes": kv_sel},
        "attend_bwd_dq": {"bytes": dq_bytes, "flops": dq_flops, "gather_bytes": kv_sel},
        "attend_bwd_dkdv": {"bytes": dkdv_bytes, "flops": dkdv_flops},
        # the work list and the partial sums are not part of the method
        "attend_bwd_finalize": {"bytes": 0.0, "flops": 0.0},
    }


PMC_SUMMARIES = {"qwen3_8b_layer_ctx16k": os.path.join(ROOT, "profiles", "hga_step_ctx16k_hbm_traffic.json"),
                 "planted_b8_ctx32k": os.path.join(ROOT, "profiles", "hga_step_planted_b8_ctx32k_hbm_traffic.json"),
                 "decode_b8_ctx32k": os.path.join(ROOT, "profiles", "hga_decode_ctx32k_hbm_traffic.json")}
MFMA_SUMMARIES = {"qwen3_8b_layer_ctx16k": os.path.join(ROOT, "profiles", "hga_step_ctx16k_mfma.json")}
STALL_SUMMARIES = {"qwen3_8b_layer_ctx16k": os.path.join(ROOT, "profiles", "hga_step_ctx16k_stalls.json")}
CSRC = os.path.join(ROOT, "sparse_long_context_hga_amd", "csrc")
# kernel-name prefix -> step kernel (first match wins)
KERNEL_KEYS = [("summaries_kernel", "summaries"), ("route_attend_", "route_attend"), ("route_", "route"),
               ("attend_fwd_", "attend_fwd"),
               ("attend_bwd_dq_", "attend_bwd_dq"),
               ("attend_bwd_dkdv_finalize", "attend_bwd_finalize"), ("attend_bwd_dkdv_", "attend_bwd_dkdv"),
               ("decode_route_kernel", "decode_route"), ("decode_attend_kernel", "decode_attend")]


def _short_name(name):
    import re
    name = name.replace("void ", "").replace("hga::(anonymous namespace)::", "")
    return re.split(r"\((?!anonymous)", name, maxsplit=1)[0]


def traffic_summary(fetch_csv, write_csv, calib_mib, workload):
    """Per-launch HBM bytes of each step kernel from two counter passes.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by the factor
    that makes the calibration scale-copy kernel (torch.mul of `calib_mib` MiB
    of fp32; reads and writes exactly that many bytes) read its known size.
    For each kernel the count over the step dispatches is averaged (the history
    summaries, built once outside the step, are a different grid and dropped)."""
    import csv
    import collections
    n = calib_mib * (1 << 20)
    out = {"workload": workload, "source_sha256": kernel_source_digest(workload), "calibration_bytes": n,
           "kernels": {}}
    per = {}
    for label, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = list(csv.DictReader(open(path)))
        calib = [float(r["Counter_Value"]) * 1024 for r in rows if "AUnaryFunctor" in r["Kernel_Name"]]
        if len(calib) != 1:
            raise SystemExit(f"{path}: expected one calibration scale-copy dispatch, found {len(calib)}")
        factor = n / calib[0]
        out[f"{label}_factor"] = round(factor, 5)
        groups = collections.defaultdict(list)
        for r in rows:
            short = _short_name(r["Kernel_Name"])
            key = next((k for pre, k in KERNEL_KEYS if short.startswith(pre)), None)
            if key is not None:
                groups[(key, r["Grid_Size"])].append(float(r["Counter_Value"]) * 1024 * factor)
        for (key, _grid), vals in groups.items():
            prev = per.get((key, label))
            if prev is None or len(vals) > len(prev):          # the step's dispatches are the most frequent
                per[(key, label)] = vals
    for (key, label), vals in sorted(per.items()):
        k = out["kernels"].setdefault(key, {})
        k[f"{label}_bytes_per_launch"] = round(statistics.mean(vals))
        k["launches"] = len(vals)
    for k in out["kernels"].values():
        k["hbm_bytes_per_launch"] = k.get("fetch_bytes_per_launch", 0) + k.get("write_bytes_per_launch", 0)
    return out


def mfma_summary(counter_csv, workload):
    """Matrix-core use of each step kernel from one counter pass (rocprofv3 derived
    counters, per dispatch): MfmaUtil = busy cycles of the MFMA units over (GPU
    active cycles x SIMDs), in percent; MfmaFlopsBF16 = bf16 MFMA operations x 512
    flops, as the hardware counts them (masked and padded work included).  Averaged
    over the step's dispatches of each kernel (most frequent grid)."""
    import csv
    import collections
    out = {"workload": workload, "source_sha256": kernel_source_digest(workload), "kernels": {}}
    groups = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(counter_csv)):
        short = _short_name(r["Kernel_Name"])
        key = next((k for pre, k in KERNEL_KEYS if short.startswith(pre)), None)
        if key is None:
            continue
        groups[(key, r["Grid_Size"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    best = {}
    for (key, _grid), cnt in groups.items():
        n = len(cnt.get("MfmaUtil", []))
        if key not in best or n > best[key][0]:
            best[key] = (n, cnt)
    for key, (n, cnt) in sorted(best.items()):
        out["kernels"][key] = {
            "launches": n,
            "mfma_util_pct": round(statistics.mean(cnt["MfmaUtil"]), 2) if cnt.get("MfmaUtil") else None,
            "mfma_bf16_flops_per_launch": round(statistics.mean(cnt["MfmaFlopsBF16"]))
            if cnt.get("MfmaFlopsBF16") else None,
        }
    return out


def stall_summary(counter_csvs, workload):
    """Where each step kernel's waves spend their time, from SQ counter passes (per
    dispatch, averaged over the step's dispatches of each kernel).  The wave-cycle
    counters (SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_*) share
    one unit (4 cycles), so their ratios are fractions of the waves' lifetime:
    waiting on an s_waitcnt or a data dependency (SQ_WAIT_ANY), ready but not issued
    because the unit or the issue slot is taken (SQ_WAIT_INST_ANY), and issuing each
    instruction type (SQ_ACTIVE_INST_*).  SQ_VALU_MFMA_COEXEC_CYCLES over
    SQ_VALU_MFMA_BUSY_CYCLES is the share of matrix-busy cycles in which a vector
    instruction issued as well."""
    import csv
    import collections
    groups = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in counter_csvs:
        for r in csv.DictReader(open(path)):
            short = _short_name(r["Kernel_Name"])
            key = next((k for pre, k in KERNEL_KEYS if short.startswith(pre)), None)
            if key is not None:
                groups[(key, r["Grid_Size"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    best = {}
    for (key, _grid), cnt in groups.items():
        n = max(len(v) for v in cnt.values())
        if key not in best or n > best[key][0]:
            best[key] = (n, cnt)
    out = {"workload": workload, "source_sha256": kernel_source_digest(workload), "kernels": {}}
    for key, (_n, cnt) in sorted(best.items()):
        m = {c: statistics.mean(v) for c, v in cnt.items()}
        k = {"launches": max(len(v) for v in cnt.values()), "counters_per_launch": {c: round(v) for c, v in m.items()}}
        wc = m.get("SQ_WAVE_CYCLES")
        if wc:
            for c, label in (("SQ_WAIT_ANY", "wait_dependency"), ("SQ_WAIT_INST_ANY", "wait_issue"),
                             ("SQ_ACTIVE_INST_ANY", "active_any"), ("SQ_ACTIVE_INST_VALU", "active_valu"),
                             ("SQ_ACTIVE_INST_LDS", "active_lds"), ("SQ_ACTIVE_INST_SCA", "active_scalar"),
                             ("SQ_WAIT_INST_LDS", "wait_issue_lds")):
                if c in m:
                    k[f"{label}_frac"] = round(m[c] / wc, 4)
        if m.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            k["valu_coissue_frac_of_mfma_busy"] = round(m.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0)
                                                        / m["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
        if m.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in m:
            k["lds_bank_conflict_frac"] = round(m["SQ_LDS_BANK_CONFLICT"] / m["SQ_LDS_IDX_ACTIVE"], 4)
        out["kernels"][key] = k
    return out


def measured_mfma(kernel, workload, ms):
    """Counter figures of `kernel` from the committed MFMA summary, with the hardware
    bf16 MFMA rate over the HIP-event duration `ms`; None when no summary exists for
    this workload or the kernels changed since it was taken."""
    try:
        with open(MFMA_SUMMARIES[workload]) as f:
            summ = json.load(f)
    except (KeyError, OSError, ValueError):
        return None
    if summ.get("workload") != workload or summ.get("source_sha256") != kernel_source_digest(workload):
        return None
    k = summ.get("kernels", {}).get(kernel)
    if k is None or k.get("mfma_bf16_flops_per_launch") is None:
        return None
    tfl = k["mfma_bf16_flops_per_launch"] / (ms * 1e-3) / 1e12
    return {"util_pct": k.get("mfma_util_pct"), "hw_bf16_tflops": round(tfl, 2),
            "frac_of_peak": round(tfl / BF16_PEAK_TFLOPS, 4)}


# Kernel sources each measured workload runs (device headers included).
WORKLOAD_SOURCES = {
    "qwen3_8b_layer_ctx16k": ["summaries.hip", "route.hip", "attend_fwd.hip", "attend_bwd.hip", "hga_device.h",
                              "hga_select.h", "route_phase.h"],
    "planted_b8_ctx32k": ["summaries.hip", "route.hip", "attend_fwd.hip", "attend_bwd.hip", "hga_device.h",
                          "hga_select.h", "route_phase.h"],
    "decode_b8_ctx32k": ["decode.hip", "summaries.hip", "hga_device.h", "hga_select.h"],
}


def _code_only(text):
    """C++ source without comments and with every whitespace run folded to one
    space (string and character literals kept as they are)."""
    import re
    tok = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)
    text = tok.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return " ".join(text.split())


def kernel_source_digest(workload):
    """sha256 over the code of the kernel sources the workload runs (comments and
    layout left out): counter figures are only valid for this exact code."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(WORKLOAD_SOURCES[workload]):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), or None when no
    summary exists for this workload or the kernels changed since it was taken."""
    try:
        with open(PMC_SUMMARIES[workload]) as f:
            summ = json.load(f)
    except (KeyError, OSError, ValueError):
        return None
    if summ.get("workload") != workload or summ.get("source_sha256") != kernel_source_digest(workload):
        return None
    k = summ.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def make_workload(name):
    import hga_inputs as hi
    return {"qwen3_8b_layer_ctx16k": hi.qwen_16k, "qwen3_8b_layer_ctx4k": hi.qwen_2k_hist,
            "planted_b8_ctx32k": hi.planted_batch}[name]()


def achievable_rates(seconds=0.15):
    """What this machine reaches on plain library work, for context next to the spec
    peaks: a device copy of 512 MiB (torch copy_: reads and writes 512 MiB) and a
    dense 8192^3 bf16 GEMM (torch.matmul, hipBLASLt); the best of repetitions run
    for about `seconds` each (at least 10) after 3 warm-ups.  Run before a
    benchmark's warm-up steps, this sustained load also brings the core clock from
    idle to the level it holds under load."""
    import torch
    mk = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731

    def best(fn):
        for _ in range(3):
            fn()
        ts = []
        t_end = time.perf_counter() + seconds
        while len(ts) < 10 or time.perf_counter() < t_end:
            e0, e1 = mk(), mk()
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts), len(ts)
    n = 512 << 20
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    t_copy, n_copy = best(lambda: y.copy_(x))
    copy_gbs = 2 * n / t_copy / 1e9
    del x, y
    m = 8192
    a = torch.randn(m, m, device="cuda", dtype=torch.bfloat16).contiguous()
    b = torch.randn(m, m, device="cuda", dtype=torch.bfloat16).contiguous()
    t_gemm, n_gemm = best(lambda: torch.matmul(a, b))
    gemm_tfs = 2 * m ** 3 / t_gemm / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": round(copy_gbs, 1), "bf16_gemm_TFLOPs": round(gemm_tfs, 1),
            "how": f"best of {n_copy} torch copy_ of 512 MiB (bytes read + written) and of {n_gemm} torch.matmul "
                   f"8192^3 bf16, each repeated for about {seconds} s"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------------ CPU oracle leg
def cpu_baseline(w, q_prev=None, min_seconds=10.0, max_reps=5):
    """The CPU oracle, as it stands, on the same step (all of it), repeated until
    about `min_seconds` of work; returns tokens/s from the median repetition."""
    import numpy as np
    from oracle import hga_oracle as ora
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    B, H, T, d = w.k_cache.shape
    gs = np.zeros((B, H, T // 8, d), np.float32)
    cs = np.zeros((B, H, T // 64, d), np.float32)
    ora.build_summaries(w.k_cache, 0, w.t_hist, w.dtype, gs, cs)   # history: untimed, as on the GPU
    times = []
    t_all = time.perf_counter()
    while len(times) < max_reps and (time.perf_counter() - t_all) < min_seconds:
        t0 = time.perf_counter()
        ora.build_summaries(w.k_cache, w.t_hist, w.t_hist + w.seg_len, w.dtype, gs, cs)
        if q_prev is None:
            _, gidx, _ = ora.route(w.q, cs, gs, w.t_hist, w.seg_len, w.top_chunks, w.top_groups, w.group_size)
        else:
            _, gidx, _ = ora.route_causal(w.q, q_prev, cs, gs, w.t_hist, w.seg_len, w.top_chunks, w.top_groups,
                                          w.group_size)
        ora.attend_fwd(w.q, w.k_cache, w.v_cache, w.t_hist, gidx, w.softmax_scale, w.group_size)
        if w.d_o is not None:
            ora.attend_bwd(w.q, w.k_cache, w.v_cache, w.d_o, w.t_hist, gidx, w.softmax_scale, w.group_size)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": w.batch * w.seg_len / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"the full step of this workload (active summaries, route, forward, backward), "
                      f"{len(times)} repetitions, median {t:.2f} s"}


# ------------------------------------------------------------------ generation
def decode_metric(t_cap):
    return (f"HGA decode tokens/s at {t_cap // 1024}K ctx (one new token per sequence per step); "
            f"% of HBM roofline")


def decode_work(w, cidx, gidx):
    """Algorithmic HBM bytes of the two generation kernels for one step: routing reads
    the query heads, every candidate chunk summary and the selected chunks' group
    summaries and writes the selection; attention reads the query heads and the K
    and V rows of every attended token, writes O and LSE, and the summaries of each
    chunk that a new token completes."""
    import numpy as np
    B, Hq, Hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    el = 2 if w.dtype == "bf16" else 4
    pos = np.asarray(w.pos)
    live = pos >= 0
    J = np.where(live, pos // 64, 0)
    q_bytes = int(live.sum()) * Hq * d * el
    nc = (cidx >= 0).sum(axis=-1)                     # [B, Hkv]
    ng = (gidx >= 0).sum(axis=-1)
    route = q_bytes + Hkv * int(J.sum()) * d * el + int((8 * nc).sum()) * d * el + (cidx.size + gidx.size) * 4
    local = np.where(live, pos - 64 * J + 1, 0)
    tokens = int((8 * ng).sum()) + Hkv * int(local.sum())
    done = int(((pos + 1) % 64 == 0)[live].sum()) * Hkv * 9 * d * el
    attend = q_bytes + tokens * d * el * 2 + q_bytes + int(live.sum()) * Hq * 4 + gidx.size * 4 + done
    return {"decode_route": {"bytes": float(route), "flops": 0.0},
            "decode_attend": {"bytes": float(attend), "flops": 0.0}}


def cpu_baseline_decode(w, min_seconds=10.0, max_reps=50):
    """The CPU oracle on the same generation step (route, attention, summary update)."""
    import numpy as np
    from oracle import hga_oracle as ora
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    B, H, T, d = w.k_cache.shape
    gs = np.zeros((B, H, T // 8, d), np.float32)
    cs = np.zeros((B, H, T // 64, d), np.float32)
    ora.build_summaries(w.k_cache, 0, T, w.dtype, gs, cs)            # the prompt: untimed, as on the GPU
    times = []
    t_all = time.perf_counter()
    while len(times) < max_reps and (time.perf_counter() - t_all) < min_seconds:
        t0 = time.perf_counter()
        _, gidx, _ = ora.decode_route(w.q, cs, gs, w.pos, w.top_chunks, w.top_groups, w.group_size)
        ora.decode_attend(w.q, w.k_cache, w.v_cache, w.pos, gidx, w.softmax_scale, w.group_size)
        ora.decode_summaries(w.k_cache, w.pos, w.dtype, gs, cs)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    n_tok = int((np.asarray(w.pos) >= 0).sum())
    return {"value": n_tok / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the full generation step of this workload ({n_tok} tokens: route, attention, summary "
                      f"update), {len(times)} repetitions, median {t * 1e3:.1f} ms"}


def main_decode(args):
    import numpy as np
    import torch
    import hga_inputs as hi
    import sparse_long_context_hga_amd as hga

    w = {"decode_b8_ctx32k": hi.decode_b8_ctx32k, "decode_b64_ctx16k": hi.decode_b64_ctx16k}[args.workload]()
    print(f"[bench] workload {w.name}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim} "
          f"t_cap={w.t_cap} pos={list(w.pos)} k_c={w.top_chunks} k_g={w.top_groups}", file=sys.stderr, flush=True)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = lambda x: torch.from_numpy(x).to("cuda").to(dt).contiguous()   # noqa: E731
    shape = hga.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.top_chunks, w.top_groups,
                           w.dtype, w.softmax_scale)
    q, k, v = dev(w.q), dev(w.k_cache), dev(w.v_cache)
    B, Hkv, T, d = k.shape
    gsum = torch.zeros(B, Hkv, T // 8, d, dtype=dt, device="cuda")
    csum = torch.zeros(B, Hkv, T // 64, d, dtype=dt, device="cuda")
    pos = torch.tensor(w.pos, dtype=torch.int32, device="cuda")
    cidx = torch.empty(B, Hkv, w.top_chunks, dtype=torch.int32, device="cuda")
    gidx = torch.empty(B, Hkv, w.top_groups, dtype=torch.int32, device="cuda")
    o = torch.empty(B, w.n_q_heads, d, dtype=dt, device="cuda")
    lse = torch.empty(B, w.n_q_heads, dtype=torch.float32, device="cuda")
    ws = torch.zeros(hga.hga_decode_workspace_size(shape, T), dtype=torch.uint8, device="cuda")
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] calibration: fill then scale-copy of {n} bytes", file=sys.stderr, flush=True)
        del src, dst
    hga.hga_build_summaries(shape, k, T, 0, T, gsum, csum)    # the prompt's summaries: untimed
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    mk = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    # timing marks go on extra steps after the timed region (ids args.steps ...)
    marked = list(range(args.steps, args.steps + max(1, args.marked_steps)))
    ev = {i: [mk() for _ in range(3)] for i in marked}
    for e in [x for i in marked for x in ev[i]]:
        e.record(stream)
    torch.cuda.synchronize()

    def step(i):
        se = ev.get(i)
        if se: se[0].record(stream)
        hga.hga_decode_route(shape, q, csum, gsum, T, pos, cidx, gidx, ws)
        if se: se[1].record(stream)
        hga.hga_decode_attend(shape, q, k, v, T, pos, gidx, o, lse, ws, gsum, csum)
        if se: se[2].record(stream)

    for i in range(args.warmup):
        step(-1 - i)
    torch.cuda.synchronize()
    if args.cold:
        # every step's inputs leave the MALL first: 512 MiB written between steps,
        # outside the step's own events
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        sev = [(mk(), mk()) for _ in range(args.steps)]
        for i in range(args.steps):
            flush.fill_(i & 255)
            sev[i][0].record(stream)
            step(i)
            sev[i][1].record(stream)
        torch.cuda.synchronize()
        ms_per_step = statistics.mean(a.elapsed_time(b) for a, b in sev)
    else:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / args.steps
    for i in marked:
        step(i)
    torch.cuda.synchronize()
    avg = lambda pairs: statistics.mean(a.elapsed_time(b) for a, b in pairs)   # noqa: E731
    kern_ms = {"decode_route": avg((ev[i][0], ev[i][1]) for i in marked),
               "decode_attend": avg((ev[i][1], ev[i][2]) for i in marked)}
    work = decode_work(w, cidx.cpu().numpy(), gidx.cpu().numpy())
    kernels = {}
    for kname, ms in kern_ms.items():
        gbs = work[kname]["bytes"] / (ms * 1e-3) / 1e9
        kernels[kname] = {"ms": round(ms, 5), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    dom = max(kern_ms, key=lambda kk: kern_ms[kk])
    ach = work[dom]["bytes"] / (kern_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom, w.name), "kernel": dom}
    n_tok = int((np.asarray(w.pos) >= 0).sum())
    out = {
        "metric": decode_metric(w.t_cap), "value": round(n_tok / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "t_cap": w.t_cap, "positions": [int(x) for x in w.pos],
                   "top_chunks": w.top_chunks, "top_groups": w.top_groups, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "kernels": kernels,
        "kernel_timing": f"HIP events between the two calls (one kernel each) on {len(marked)} steps run after "
                         f"the timed region",
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w)
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ rollout
ROLLOUT_METRIC = "HGA rollout tokens/s (summaries + route + forward, 64 segments) at 131K ctx; % of HBM roofline"


def main_rollout(args):
    """The 131,072-token evaluation rollout: 64 segments of 2,048 tokens, each
    building its summaries, routing against all earlier segments and attending
    (forward only), with every segment's Q, K and V resident in HBM.  One step is
    the whole rollout; tokens/s = 131,072 / step time."""
    import numpy as np
    import torch
    import hga_inputs as hi
    import sparse_long_context_hga_amd as hga

    S, T, Hq, Hkv, d = hi.ROLLOUT_SEG, hi.ROLLOUT_TOKENS, 32, 8, 128
    n_seg = T // S
    print(f"[bench] workload rollout_131k: {n_seg} segments of {S} tokens, {Hq}/{Hkv}/{d}, top-16/top-64",
          file=sys.stderr, flush=True)
    shape = hga.make_shape(1, Hq, Hkv, d, 16, 64, "bf16", 1.0 / np.sqrt(d))
    dt = torch.bfloat16
    kc = torch.zeros(1, Hkv, T, d, dtype=dt, device="cuda")
    vc = torch.zeros_like(kc)
    qs = []
    for s_ in range(n_seg):
        q, k, v = hi.rollout_segment(s_)
        kc[:, :, s_ * S:(s_ + 1) * S] = torch.from_numpy(k).to(dt).cuda()
        vc[:, :, s_ * S:(s_ + 1) * S] = torch.from_numpy(v).to(dt).cuda()
        qs.append(torch.from_numpy(q).to(dt).cuda().contiguous())
    gsum = torch.zeros(1, Hkv, T // 8, d, dtype=dt, device="cuda")
    csum = torch.zeros(1, Hkv, T // 64, d, dtype=dt, device="cuda")
    nb = S // 64
    cidx = torch.empty(1, Hkv, nb, 16, dtype=torch.int32, device="cuda")
    gidx = torch.empty(1, Hkv, nb, 64, dtype=torch.int32, device="cuda")
    o = torch.empty(1, Hq, S, d, dtype=dt, device="cuda")
    lse = torch.empty(1, Hq, S, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    mk = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    ev = [[mk() for _ in range(hga.HGA_FWD_EVENTS)] for _ in range(n_seg)]

    def rollout(marks):
        for s_ in range(n_seg):
            # summaries of the segment, then routing + attention (hga_forward); the marked
            # rollout times every kernel from its own dispatch
            hga.hga_forward(shape, qs[s_], kc, vc, csum, gsum, T, s_ * S, S, cidx, gidx, o, lse,
                            events=ev[s_] if marks else None)

    for _ in range(args.warmup):
        rollout(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        rollout(False)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    rollout(True)                                   # one more, with timing marks
    torch.cuda.synchronize()
    kern_ms = {"summaries": 0.0, "route_attend": 0.0}
    for s_ in range(n_seg):
        kern_ms["summaries"] += ev[s_][0].elapsed_time(ev[s_][1])
        kern_ms["route_attend"] += ev[s_][2].elapsed_time(ev[s_][3])
    # algorithmic bytes of the whole rollout: every segment's summaries (its K read,
    # summaries written), route (Q and the candidate chunk summaries of every block,
    # the group summaries of its selected chunks) and forward (Q, gathered and own
    # K/V, O, LSE); every block selects min(16, J) chunks and then 64 groups once
    # J >= 8.
    el = 2
    work = {"summaries": 0.0, "route_attend": 0.0}
    for s_ in range(n_seg):
        work["summaries"] += Hkv * S * d * el + Hkv * (S // 8 + S // 64) * d * el
        J = np.arange(nb) + s_ * S // 64
        nc = np.minimum(16, J)
        ng = np.minimum(64, 8 * nc)
        q_bytes = Hq * S * d * el
        # routing reads the summaries; Q is read once for routing and attention
        work["route_attend"] += (q_bytes + Hkv * float(np.sum(J + 8 * nc)) * d * el + q_bytes
                                 + Hkv * float(np.sum(8 * ng)) * d * el * 2 + Hkv * nb * 64 * d * el * 2 + Hq * S * 4)
    kernels = {}
    for k_, ms in kern_ms.items():
        gbs = work[k_] / (ms * 1e-3) / 1e9
        kernels[k_] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    dom = max(kern_ms, key=lambda k_: kern_ms[k_])
    ach = work[dom] / (kern_ms[dom] * 1e-3) / 1e9
    out = {
        "metric": ROLLOUT_METRIC, "value": round(T / (ms_per_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "rollout_131k", "batch": 1, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d,
                   "segments": n_seg, "seg_len": S, "context": T, "top_chunks": 16, "top_groups": 64,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom},
        "kernels": kernels,
        "kernel_timing": "every kernel timed from its own dispatch in one extra, marked rollout (summed over the "
                         "64 segments)",
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_rollout()
    print(json.dumps(out), flush=True)


def cpu_baseline_rollout(max_reps=3, min_seconds=10.0):
    """The CPU oracle, as it stands, on a bounded sample of the rollout: the last
    segment (2,048 tokens routed over 2,016 to 2,047 candidate chunks per block,
    then attended), with every earlier segment's summaries built untimed."""
    import numpy as np
    import hga_inputs as hi
    from oracle import hga_oracle as ora
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    S, T, Hkv, d = hi.ROLLOUT_SEG, hi.ROLLOUT_TOKENS, 8, 128
    n_seg = T // S
    k_all = np.zeros((1, Hkv, T, d), np.float32)
    v_all = np.zeros((1, Hkv, T, d), np.float32)
    for s_ in range(n_seg):
        _, k, v = hi.rollout_segment(s_)
        k_all[:, :, s_ * S:(s_ + 1) * S] = k
        v_all[:, :, s_ * S:(s_ + 1) * S] = v
    q, _, _ = hi.rollout_segment(n_seg - 1)
    t_hist = (n_seg - 1) * S
    gs = np.zeros((1, Hkv, T // 8, d), np.float32)
    cs = np.zeros((1, Hkv, T // 64, d), np.float32)
    ora.build_summaries(k_all, 0, t_hist, "bf16", gs, cs)            # earlier segments: untimed
    times = []
    t_all = time.perf_counter()
    while len(times) < max_reps and (time.perf_counter() - t_all) < min_seconds:
        t0 = time.perf_counter()
        ora.build_summaries(k_all, t_hist, T, "bf16", gs, cs)
        _, gidx, _ = ora.route(q, cs, gs, t_hist, S, 16, 64, 4)
        ora.attend_fwd(q, k_all, v_all, t_hist, gidx, 1.0 / np.sqrt(d), 4)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": S / t, "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"the last segment of the rollout (summaries, route over 2,016-2,047 candidate chunks per "
                      f"block, forward), {len(times)} repetitions, median {t:.2f} s"}


# ------------------------------------------------------------------ host-RAM tier
def main_host_tier(args):
    """The layer step with the detached history in pinned host memory: the active
    segment's summaries (built in the staging cache, copied into the tables at their
    global position), routing over the tables in HBM, staging of the selected history
    groups over the host link (hga_stage_history), then the forward and backward on
    the staging cache.  Inputs are in place before timing (history in host memory,
    the segment in HBM); the step rate includes the host-link transfers."""
    import numpy as np
    import torch
    import sparse_long_context_hga_amd as hga

    w = make_workload(args.workload)
    B, Hq, Hkv, d, S, th = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seg_len, w.t_hist
    T = th + S
    nb = S // 64
    dt = torch.bfloat16
    shape = hga.make_shape(B, Hq, Hkv, d, w.top_chunks, w.top_groups, w.dtype, w.softmax_scale)
    print(f"[bench] workload {w.name}, history in host memory: B={B} Hq={Hq} Hkv={Hkv} d={d} t_hist={th} S={S}",
          file=sys.stderr, flush=True)
    k_full = torch.from_numpy(w.k_cache).to(dt)
    v_full = torch.from_numpy(w.v_cache).to(dt)
    k_host = k_full.pin_memory()
    v_host = v_full.pin_memory()
    gsum = torch.zeros(B, Hkv, T // 8, d, dtype=dt, device="cuda")
    csum = torch.zeros(B, Hkv, T // 64, d, dtype=dt, device="cuda")
    kd = k_full.cuda()                                        # history summaries: built once, untimed
    hga.hga_build_summaries(shape, kd, T, 0, th, gsum, csum)
    torch.cuda.synchronize()
    del kd
    sh = hga.hga_stage_history_min(shape, th, S)
    cap = sh + S
    k_st = torch.zeros(B, Hkv, cap, d, dtype=dt, device="cuda")
    v_st = torch.zeros_like(k_st)
    k_st[:, :, sh:] = k_full[:, :, th:T].cuda()              # the active segment: in HBM before timing
    v_st[:, :, sh:] = v_full[:, :, th:T].cuda()
    gs_seg = torch.zeros(B, Hkv, cap // 8, d, dtype=dt, device="cuda")
    cs_seg = torch.zeros(B, Hkv, cap // 64, d, dtype=dt, device="cuda")
    dev = lambda x: torch.from_numpy(x).to("cuda").to(dt).contiguous()   # noqa: E731
    q, d_o = dev(w.q), dev(w.d_o)
    cidx = torch.empty(B, Hkv, nb, w.top_chunks, dtype=torch.int32, device="cuda")
    gidx = torch.empty(B, Hkv, nb, w.top_groups, dtype=torch.int32, device="cuda")
    gst = torch.empty_like(gidx)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, S, dtype=torch.float32, device="cuda")
    dq = torch.empty_like(q)
    dk = torch.empty(B, Hkv, S, d, dtype=dt, device="cuda")
    dv = torch.empty_like(dk)
    ws = torch.empty(hga.hga_attend_bwd_workspace_size(shape, sh, S), dtype=torch.uint8, device="cuda")
    ws[:hga.HGA_BWD_WORKSPACE_CLEAR_BYTES].zero_()
    stream = torch.cuda.current_stream()
    mk = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731

    def step(ev=None):
        hga.hga_build_summaries(shape, k_st, cap, sh, sh + S, gs_seg, cs_seg)
        gsum[:, :, th // 8:T // 8].copy_(gs_seg[:, :, sh // 8:cap // 8])
        csum[:, :, th // 64:T // 64].copy_(cs_seg[:, :, sh // 64:cap // 64])
        hga.hga_route(shape, q, csum, gsum, T, th, S, cidx, gidx)
        if ev:
            ev[0].record(stream)
        hga.hga_stage_history(shape, k_host, v_host, T, th, S, gidx, k_st, v_st, cap, sh, gst)
        if ev:
            ev[1].record(stream)
        hga.hga_attend_fwd(shape, q, k_st, v_st, cap, sh, S, gst, o, lse)
        hga.hga_attend_bwd(shape, q, k_st, v_st, o, lse, d_o, cap, sh, S, gst, dq, dk, dv, ws)

    achievable = None if args.no_calibration else achievable_rates()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    n_mark = max(1, args.marked_steps)
    evs = [[mk(), mk()] for _ in range(n_mark)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    stage_ms = statistics.mean(a.elapsed_time(b) for a, b in evs)
    g = gidx.cpu().numpy()
    staged = 0
    for b in range(B):
        for h in range(Hkv):
            ids = g[b, h].ravel()
            staged += len(set(int(x) for x in ids if 0 <= x < th // 8))
    staged_bytes = staged * 8 * d * 2 * 2                      # K and V rows of every staged group
    out = {
        "metric": METRIC + " -- history in host RAM (host-link-inclusive)", "value": round(B * S / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d, "t_hist": th,
                   "seg_len": S, "top_chunks": w.top_chunks, "top_groups": w.top_groups,
                   "history": "pinned host memory; selected groups staged into HBM",
                   "staging_tokens": sh, "parallelism": "none (1 GPU)"},
        "stage": {"ms": round(stage_ms, 5), "groups_staged": staged, "bytes": staged_bytes,
                  "host_link_GB/s": round(staged_bytes / (stage_ms * 1e-3) / 1e9, 1),
                  "of_history": round(staged / (B * Hkv * th // 8), 4)},
        "achievable": achievable,
        "kernel_timing": f"staging call timed with HIP events on {n_mark} steps run after the timed region",
    }
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.mfma_summary:
        summ = mfma_summary(args.mfma_summary, args.workload)
        with open(MFMA_SUMMARIES[args.workload], "w") as f:
            json.dump(summ, f, indent=1)
        print(json.dumps(summ, indent=1))
        return
    if args.stall_summary:
        summ = stall_summary(args.stall_summary, args.workload)
        with open(STALL_SUMMARIES[args.workload], "w") as f:
            json.dump(summ, f, indent=1)
        print(json.dumps(summ, indent=1))
        return
    if args.traffic_summary:
        if not args.copy_calibration_mib:
            raise SystemExit("--traffic-summary needs the --copy-calibration-mib of the profiled run")
        summ = traffic_summary(*args.traffic_summary, args.copy_calibration_mib, args.workload)
        with open(PMC_SUMMARIES[args.workload], "w") as f:
            json.dump(summ, f, indent=1)
        print(json.dumps(summ, indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the HGA layer path has no multi-GPU mode (it would shard "
              "by sequence and KV head, with no communication inside the layer).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import sparse_long_context_hga_amd as hga
    from sparse_long_context_hga_amd.layer import HGALayerBuffers

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    hga.lib()
    if args.workload.startswith("decode"):
        return main_decode(args)
    if args.workload == "rollout_131k":
        return main_rollout(args)
    if args.history == "host":
        return main_host_tier(args)
    w = make_workload(args.workload)
    print(f"[bench] workload {w.name}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim} "
          f"t_hist={w.t_hist} S={w.seg_len} k_c={w.top_chunks} k_g={w.top_groups}", file=sys.stderr, flush=True)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = lambda x: torch.from_numpy(x).to("cuda").to(dt).contiguous()   # noqa: E731
    shape = hga.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.top_chunks, w.top_groups,
                           w.dtype, w.softmax_scale)
    L = HGALayerBuffers(shape, dev(w.q), dev(w.k_cache), dev(w.v_cache), w.t_hist,
                        dev(w.d_o) if w.d_o is not None else None)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")   # fill kernel: writes n bytes
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)                                     # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(f"[bench] calibration: fill then scale-copy of {n} bytes", file=sys.stderr, flush=True)
        del src, dst
    q_prev_np = None
    if args.routing == "causal":
        import hga_inputs as hi
        q_prev_np = hi.prev_query_block(seed=1, batch=w.batch, n_q_heads=w.n_q_heads, head_dim=w.head_dim,
                                        dtype=w.dtype)
        q_prev = dev(q_prev_np)
    L.summaries(0, w.t_hist)                                  # history summaries: built once, untimed
    torch.cuda.synchronize()
    # What the box reaches on plain library work; these sustained copies and GEMMs
    # also bring the core clock up from idle before the warm-up steps.
    achievable = None if args.no_calibration else achievable_rates()

    stream = torch.cuda.current_stream()
    mk = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    n_bwd = hga.HGA_BWD_KERNELS

    def step(fev=None, bev=None):
        if args.routing == "causal":
            L.forward_causal(q_prev, events=fev)      # summaries, then causal routing + attention
        else:
            L.forward(events=fev)                     # summaries, then routing + attention
        if L.do is not None:
            L.bwd(events=bev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.cold:
        # every step's inputs leave the MALL first: 512 MiB written between steps,
        # outside the step's own events
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        sev = [(mk(), mk()) for _ in range(args.steps)]
        for i in range(args.steps):
            flush.fill_(i & 255)
            sev[i][0].record(stream)
            step()
            sev[i][1].record(stream)
        torch.cuda.synchronize()
        ms_per_step = statistics.mean(a.elapsed_time(b) for a, b in sev)
    else:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / args.steps

    # Per-kernel times: after the timed region, marked steps in which every kernel is
    # timed from its own dispatch (start / stop events recorded by the launches, on the
    # stream the library launches on); with --cold each is preceded by the flush too.
    n_mark = max(1, args.marked_steps)
    fev = [[mk() for _ in range(hga.HGA_FWD_EVENTS)] for _ in range(n_mark)]
    bev = [[mk() for _ in range(2 * n_bwd)] for _ in range(n_mark)]
    for i in range(n_mark):
        if args.cold:
            flush.fill_(i & 255)
        step(fev[i], bev[i])
    torch.cuda.synchronize()
    avg = lambda pairs: statistics.mean(a.elapsed_time(b) for a, b in pairs)   # noqa: E731
    kern_ms = {"summaries": avg((e[0], e[1]) for e in fev),
               "route_attend_causal" if args.routing == "causal" else "route_attend": avg((e[2], e[3]) for e in fev)}
    if L.do is not None:
        for k, name in enumerate(("attend_bwd_dq", "attend_bwd_dkdv", "attend_bwd_finalize")):
            kern_ms[name] = avg((e[2 * k], e[2 * k + 1]) for e in bev)

    gidx = L.gidx.cpu().numpy()
    work = algorithmic_work(w, gidx)
    kernels = {}
    for k, ms in kern_ms.items():
        wk = work.get(k, {"bytes": 0.0, "flops": 0.0})
        gbs = wk["bytes"] / (ms * 1e-3) / 1e9
        tfl = wk["flops"] / (ms * 1e-3) / 1e12
        kernels[k] = {"ms": round(ms, 5), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                      "TFLOP/s": round(tfl, 2), "mfma_frac": round(tfl / BF16_PEAK_TFLOPS, 4)}
        if "gather_bytes" in wk:
            kernels[k]["gather_GB/s"] = round(wk["gather_bytes"] / (ms * 1e-3) / 1e9, 1)
        if args.routing == "block" and not args.cold:
            mc = measured_mfma(k, args.workload, ms)
            if mc is not None:
                kernels[k]["mfma_counters"] = mc
    dom = max(kern_ms, key=lambda k: kern_ms[k])
    wk = work.get(dom, {"bytes": 0.0, "flops": 0.0})
    intensity = wk["flops"] / max(wk["bytes"], 1.0)
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity >= ridge:
        ach = wk["flops"] / (kern_ms[dom] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
    else:
        ach = wk["bytes"] / (kern_ms[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4)}
    roofline["traffic"] = measured_traffic(dom, args.workload) if args.routing == "block" and not args.cold else None
    roofline["kernel"] = dom
    if achievable is not None:
        roofline["frac_of_achievable"] = round(
            ach / (achievable["hbm_copy_GBps"] if roofline["bound"] == "hbm" else achievable["bf16_gemm_TFLOPs"]), 4)

    tokens = w.batch * w.seg_len
    out = {
        "metric": METRIC, "value": round(tokens / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "t_hist": w.t_hist,
                   "seg_len": w.seg_len, "context": w.t_hist + w.seg_len, "top_chunks": w.top_chunks,
                   "top_groups": w.top_groups, "routing": args.routing,
                   "mall": "flushed before every step (512 MiB written)" if args.cold else "warm",
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "achievable": achievable,
        "kernels": kernels,
        "kernel_timing": (f"every kernel timed from its own dispatch (HIP events recorded by the launch) in "
                          f"{n_mark} steps run after the timed region" if args.routing == "block" else
                          f"HIP events between the calls (one kernel each) on the library's stream, in {n_mark} "
                          f"steps run after the timed region"),
        "kernel_sum_ms": round(sum(kern_ms.values()), 5),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q_prev_np)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
