"""CPU oracle for Hierarchical Global Attention (HGA) routed attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What HGA computes (source pages: "Long-Context Fine-Tuning with Limited VRAM",
arXiv 2607.15105 -- the adnankhan.ai note, section "Raw Abstract / Excerpt";
the seventnews article, section "HGA的不同之处" (how HGA differs); the
gist.science summary, section "解决方案" (the solution)):

  * the causal history is cut into 64-token chunks, each represented by a
    compact summary vector, and each chunk into 8-token groups with their own
    summaries;
  * a query block scores the chunk summaries with its projected queries (no
    learned router weights), keeps the top-k chunks, opens them at group level
    and keeps the top groups;
  * exact attention then runs over the exact-token K/V of the selected groups;
    summaries never act as values;
  * only the active segment is differentiable: detached history K/V receives
    no gradient (segment-wise backprop; seventnews, same section; the abstract).

Where the pages leave a step open, this file takes the readings listed below
(each one is also listed in the design notes):

  R-sum    summary = mean of the keys of the group / chunk, accumulated in fp32
           in a fixed pairwise tree (group: ((x0+x1)+(x2+x3))+((x4+x5)+(x6+x7));
           chunk: the same tree over the 8 unscaled group sums), scaled by
           1/8 resp. 1/64 and stored in the key dtype (bf16: round to nearest
           even).
  R-score  per-row score = q . summary (unscaled dot product), rounded to fp32;
           the block score is the maximum over the block's 64 positions and the
           G query heads that share the KV head.  Routing is per
           (sequence, KV head, 64-token query block).
  R-cand   candidate chunks for block j are every complete chunk before it:
           chunks 0 .. J-1 with J = t_hist/64 + j (history and earlier chunks
           of the active segment).
  R-group  candidate groups are the 8 groups of every selected chunk; one
           global top-k over them.
  R-topk   selection sorts by (score descending, index ascending), keeps
           min(k, #candidates), and stores indices ascending, padded with -1.
  R-local  besides the selected groups, each query attends to its own chunk
           causally (positions 64J .. its own position).
  R-scale  logits = softmax_scale * q . k;  LSE = natural log of sum exp(logits).
  R-grad   no gradient reaches history tokens, the summaries or the selection.
  R-causal (the strictly causal variant the seventnews article, section
           "一个真正的警告：因果泄露", says is in development; the pages give no
           design) a block is routed by the rows of the query block just before
           it instead of its own, with the same candidates (chunks 0 .. J-1) and
           the same group step.  Every input of the decision then lies before the
           block's first position, so no row can learn about later tokens from
           which chunks were chosen.  The first block of a segment uses the last
           query block of the previous segment; the very first block of a
           sequence has no candidates either way.
  R-decode (generation: the abstract on the adnankhan.ai note, "Raw Abstract /
           Excerpt", and the seventnews section "检索：密集基线无退化" say HGA can
           generate and that a serving implementation is in development; the
           pages give no design) one new token per sequence at position pos:
           its query block is that single position, so its rows are the G query
           heads of the token; candidates are chunks 0 .. J-1 with J = pos // 64;
           it attends the selected groups plus its own chunk up to and including
           itself (positions 64J .. pos).  The routing is per token, so it is
           strictly causal by construction.  When pos is the last position of a
           chunk, that chunk's group and chunk summaries are built (R-sum) so the
           next tokens can select it.  A negative pos marks an idle batch slot:
           nothing selected, O = 0, LSE = -inf.

Precision: inputs are float32 arrays whose values are exact in the workload
dtype.  Everything is computed in float64 except the two pinned rounding
points above (summaries; fp32 scores that decide the selection).

Parity pins for every function live in tests/test_oracle_*.py.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

CHUNK = 64
GROUP = 8
QBLOCK = 64
GROUPS_PER_CHUNK = CHUNK // GROUP


# ---------------------------------------------------------------------------
# Storage rounding used by R-sum (oracle's own implementation)
# ---------------------------------------------------------------------------

def _to_bf16_nearest_even(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    keep = bits >> 16
    rem = bits & 0xFFFF
    round_up = (rem > 0x8000) | ((rem == 0x8000) & ((keep & 1) == 1))
    keep = keep + round_up.astype(np.uint64)
    return (keep << 16).astype(np.uint32).view(np.float32)


# ---------------------------------------------------------------------------
# Summaries (seventnews "HGA的不同之处": 64-token chunks each kept as a compact
# summary vector, 8-token groups inside; gist.science "解决方案": summary cards per
# chunk and a summary cache for the groups).  Formula: reading R-sum.
# ---------------------------------------------------------------------------

def _pair_tree8(x: Sequence[np.ndarray]) -> np.ndarray:
    """((x0+x1)+(x2+x3)) + ((x4+x5)+(x6+x7)) in float32."""
    a = (x[0] + x[1]) + (x[2] + x[3])
    b = (x[4] + x[5]) + (x[6] + x[7])
    return a + b


def build_summaries(k_cache: np.ndarray, t_begin: int, t_end: int, dtype: str,
                    group_sum: np.ndarray, chunk_sum: np.ndarray) -> None:
    """Fill group_sum[:, :, t_begin/8 : t_end/8] and chunk_sum[:, :, t_begin/64 : t_end/64]
    from k_cache[B, Hkv, t_cap, d] (float32 values).  t_begin, t_end multiples of 64."""
    assert t_begin % CHUNK == 0 and t_end % CHUNK == 0
    for c in range(t_begin // CHUNK, t_end // CHUNK):
        gs_unscaled = []
        for u in range(GROUPS_PER_CHUNK):
            gamma = c * GROUPS_PER_CHUNK + u
            rows = [k_cache[:, :, gamma * GROUP + r, :].astype(np.float32) for r in range(GROUP)]
            s = _pair_tree8(rows)
            gs_unscaled.append(s)
            g = s * np.float32(0.125)
            group_sum[:, :, gamma, :] = _to_bf16_nearest_even(g) if dtype == "bf16" else g
        cs = _pair_tree8(gs_unscaled) * np.float32(1.0 / 64.0)
        chunk_sum[:, :, c, :] = _to_bf16_nearest_even(cs) if dtype == "bf16" else cs


# ---------------------------------------------------------------------------
# Routing (seventnews "HGA的不同之处": queries score the summaries, keep the
# top-k chunks, open them at group level; no learned router weights.
# Block-level decision from several query positions: seventnews "因果泄露").
# ---------------------------------------------------------------------------

def block_rows(q: np.ndarray, b: int, kvh: int, j: int, group_size: int) -> np.ndarray:
    """Query rows of (sequence b, KV head kvh, block j): the G heads sharing the
    KV head times the 64 positions of the block, as float64 [G*64, d]
    (row index = head_offset * 64 + position)."""
    h0 = kvh * group_size
    blk = q[b, h0:h0 + group_size, j * QBLOCK:(j + 1) * QBLOCK, :]
    return blk.reshape(-1, q.shape[-1]).astype(np.float64)


def block_scores(rows: np.ndarray, summaries: np.ndarray) -> np.ndarray:
    """R-score: max over rows of fl32(q . s) for each summary row s."""
    if summaries.shape[0] == 0:
        return np.zeros((0,), np.float32)
    per_row = (rows @ summaries.astype(np.float64).T).astype(np.float32)
    return per_row.max(axis=0)


def select_topk(scores: np.ndarray, ids: Sequence[int], k: int) -> List[int]:
    """R-topk: keep min(k, n) entries by (score desc, id asc); return them ascending."""
    order = sorted(range(len(ids)), key=lambda i: (-float(scores[i]), int(ids[i])))
    return sorted(int(ids[i]) for i in order[:max(0, min(k, len(ids)))])


def route_rows(rows, chunk_sum, group_sum, J, b, kvh, top_chunks, top_groups):
    """Two-level selection for one (sequence b, KV head kvh) over candidate chunks
    [0, J), scored by the given query rows [R, d]: returns
    (chunk_sel, group_sel, chunk_scores[J], group_ids, group_scores)."""
    sig = block_scores(rows, chunk_sum[b, kvh, :J])
    chunk_sel = select_topk(sig, list(range(J)), top_chunks)
    gids = [c * GROUPS_PER_CHUNK + u for c in chunk_sel for u in range(GROUPS_PER_CHUNK)]
    tau = block_scores(rows, group_sum[b, kvh, gids]) if gids else np.zeros((0,), np.float32)
    group_sel = select_topk(tau, gids, top_groups)
    return chunk_sel, group_sel, sig, gids, tau


def route_unit(q, chunk_sum, group_sum, t_hist, b, kvh, j, top_chunks, top_groups, group_size):
    """One (sequence, KV head, query block), routed by the block's own rows."""
    J = t_hist // CHUNK + j
    return route_rows(block_rows(q, b, kvh, j, group_size), chunk_sum, group_sum, J, b, kvh,
                      top_chunks, top_groups)


def causal_routing_rows(q, q_prev, b, kvh, j, group_size):
    """R-causal: the rows that route block j are those of the query block just
    before it -- block j-1 of this segment, or for j = 0 the last block of the
    previous segment, q_prev [B, Hq, 64, d]."""
    if j > 0:
        return block_rows(q, b, kvh, j - 1, group_size)
    return block_rows(q_prev, b, kvh, 0, group_size)


def route_unit_causal(q, q_prev, chunk_sum, group_sum, t_hist, b, kvh, j, top_chunks, top_groups,
                      group_size):
    """One unit under strictly causal routing (R-causal).  With no earlier chunk
    (J = 0) there is nothing to select and no routing rows are needed."""
    J = t_hist // CHUNK + j
    if J == 0:
        return [], [], np.zeros((0,), np.float32), [], np.zeros((0,), np.float32)
    rows = causal_routing_rows(q, q_prev, b, kvh, j, group_size)
    return route_rows(rows, chunk_sum, group_sum, J, b, kvh, top_chunks, top_groups)


def _route_all(unit_fn, B, Hkv, seg_len, top_chunks, top_groups):
    nb = seg_len // QBLOCK
    cidx = np.full((B, Hkv, nb, top_chunks), -1, np.int32)
    gidx = np.full((B, Hkv, nb, top_groups), -1, np.int32)
    tables = {}
    for b in range(B):
        for kvh in range(Hkv):
            for j in range(nb):
                cs, gs, sig, gids, tau = unit_fn(b, kvh, j)
                cidx[b, kvh, j, :len(cs)] = cs
                gidx[b, kvh, j, :len(gs)] = gs
                tables[(b, kvh, j)] = (sig, gids, tau)
    return cidx, gidx, tables


def route(q, chunk_sum, group_sum, t_hist, seg_len, top_chunks, top_groups, group_size):
    """All units.  Returns chunk_idx [B,Hkv,nb,k_c], group_idx [B,Hkv,nb,k_g] (int32,
    ascending, -1 padded) and a dict of per-unit score tables."""
    B, Hkv = chunk_sum.shape[:2]
    return _route_all(lambda b, kvh, j: route_unit(q, chunk_sum, group_sum, t_hist, b, kvh, j, top_chunks,
                                                   top_groups, group_size),
                      B, Hkv, seg_len, top_chunks, top_groups)


def route_causal(q, q_prev, chunk_sum, group_sum, t_hist, seg_len, top_chunks, top_groups, group_size):
    """All units under strictly causal routing (R-causal); outputs as route().
    q_prev [B, Hq, 64, d]: the last query block of the previous segment (needed
    when t_hist > 0, ignored otherwise)."""
    B, Hkv = chunk_sum.shape[:2]
    return _route_all(lambda b, kvh, j: route_unit_causal(q, q_prev, chunk_sum, group_sum, t_hist, b, kvh, j,
                                                          top_chunks, top_groups, group_size),
                      B, Hkv, seg_len, top_chunks, top_groups)


def selection_accepted(sel: Sequence[int], ids: Sequence[int], scores: np.ndarray, k: int,
                       rel: float = 1e-5) -> Tuple[bool, int]:
    """Acceptance of a candidate selection against oracle scores: the right size,
    no duplicates, every member beats every non-member by (score desc, id asc),
    except pairs whose scores are within `rel` relative of each other (counted)."""
    ids = [int(i) for i in ids]
    pos = {g: i for i, g in enumerate(ids)}
    sel = [int(s) for s in sel if s >= 0]
    k_eff = max(0, min(k, len(ids)))
    if len(sel) != k_eff or len(set(sel)) != len(sel) or any(s not in pos for s in sel):
        return False, 0
    chosen = set(sel)
    exempt = 0
    for x in sel:
        sx = float(scores[pos[x]])
        for y in ids:
            if y in chosen:
                continue
            sy = float(scores[pos[y]])
            if sx > sy or (sx == sy and x < y):
                continue
            if abs(sx - sy) <= rel * max(abs(sx), abs(sy)):
                exempt += 1
                continue
            return False, exempt
    return True, exempt


# ---------------------------------------------------------------------------
# Exact attention over the selected groups plus the own chunk (seventnews
# "HGA的不同之处": only the selected groups' exact-token K/V are loaded and
# attended; the abstract: a bounded set of exact historical tokens per block).
# ---------------------------------------------------------------------------

def key_tokens(group_sel: Sequence[int]) -> np.ndarray:
    """Token positions of the selected groups (ascending), -1 entries skipped."""
    g = [int(x) for x in group_sel if x >= 0]
    if not g:
        return np.zeros((0,), np.int64)
    return (np.asarray(g, np.int64)[:, None] * GROUP + np.arange(GROUP)[None, :]).reshape(-1)


def _unit_logits(rows, k_b, sel_tokens, J, scale):
    """Logits [R, n_sel + 64] of the block rows against the selected tokens and
    the own chunk; own-chunk entries later than the row's position are -inf."""
    d = rows.shape[1]
    local = np.arange(J * CHUNK, (J + 1) * CHUNK)
    keys = np.concatenate([k_b[sel_tokens], k_b[local]], 0).astype(np.float64) if len(sel_tokens) \
        else k_b[local].astype(np.float64)
    L = scale * (rows @ keys.T)
    n_sel = len(sel_tokens)
    pos = np.tile(np.arange(QBLOCK), rows.shape[0] // QBLOCK)       # row position in block
    causal = np.arange(CHUNK)[None, :] > pos[:, None]
    L[:, n_sel:][causal] = -np.inf
    return L, keys, local


def attend_fwd_unit(q, k_cache, v_cache, t_hist, group_sel, b, kvh, j, scale, group_size):
    """O [G*64, d] and LSE [G*64] (float64) for one unit."""
    J = t_hist // CHUNK + j
    rows = block_rows(q, b, kvh, j, group_size)
    sel = key_tokens(group_sel)
    L, _, local = _unit_logits(rows, k_cache[b, kvh], sel, J, scale)
    m = L.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(L - m).sum(axis=1))
    P = np.exp(L - lse[:, None])
    vals = np.concatenate([v_cache[b, kvh][sel], v_cache[b, kvh][local]], 0).astype(np.float64) \
        if len(sel) else v_cache[b, kvh][local].astype(np.float64)
    return P @ vals, lse


def attend_fwd(q, k_cache, v_cache, t_hist, group_idx, scale, group_size):
    B, Hq, S, d = q.shape
    Hkv = k_cache.shape[1]
    o = np.zeros((B, Hq, S, d), np.float64)
    lse = np.zeros((B, Hq, S), np.float64)
    for b in range(B):
        for kvh in range(Hkv):
            for j in range(S // QBLOCK):
                ou, lu = attend_fwd_unit(q, k_cache, v_cache, t_hist, group_idx[b, kvh, j],
                                         b, kvh, j, scale, group_size)
                h0 = kvh * group_size
                o[b, h0:h0 + group_size, j * QBLOCK:(j + 1) * QBLOCK] = ou.reshape(group_size, QBLOCK, d)
                lse[b, h0:h0 + group_size, j * QBLOCK:(j + 1) * QBLOCK] = lu.reshape(group_size, QBLOCK)
    return o, lse


# ---------------------------------------------------------------------------
# Backward for the active segment (adnankhan.ai "Raw Abstract": only the active
# segment stays differentiable, older KV is detached; seventnews "HGA的不同之处":
# the router has no weights, gradients reach the same projections as dense).
# Softmax-attention gradient, written out per unit:
#   D = sum_e dO*O ; dP_t = dO.v_t ; dS_t = P_t (dP_t - D)
#   dQ = scale * sum_t dS_t k_t ; for t >= t_hist: dV_t += P_t dO, dK_t += scale dS_t q
# ---------------------------------------------------------------------------

def _unit_grads(q, k_cache, v_cache, d_o, t_hist, group_sel, b, kvh, j, scale, group_size):
    J = t_hist // CHUNK + j
    rows = block_rows(q, b, kvh, j, group_size)
    dorows = block_rows(d_o, b, kvh, j, group_size)
    sel = key_tokens(group_sel)
    L, keys, local = _unit_logits(rows, k_cache[b, kvh], sel, J, scale)
    m = L.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(L - m).sum(axis=1))
    P = np.exp(L - lse[:, None])
    tokens = np.concatenate([sel, local]) if len(sel) else local
    vals = v_cache[b, kvh][tokens].astype(np.float64)
    O = P @ vals
    D = (dorows * O).sum(axis=1)
    dP = dorows @ vals.T
    dS = P * (dP - D[:, None])
    dq = scale * (dS @ keys)
    dv_tok = P.T @ dorows            # [n_keys, d]
    dk_tok = scale * (dS.T @ rows)   # [n_keys, d]
    return dq, tokens, dk_tok, dv_tok


def attend_bwd(q, k_cache, v_cache, d_o, t_hist, group_idx, scale, group_size):
    """dQ [B,Hq,S,d], dK_active / dV_active [B,Hkv,S,d] (float64)."""
    B, Hq, S, d = q.shape
    Hkv = k_cache.shape[1]
    dq = np.zeros((B, Hq, S, d), np.float64)
    dk = np.zeros((B, Hkv, S, d), np.float64)
    dv = np.zeros((B, Hkv, S, d), np.float64)
    for b in range(B):
        for kvh in range(Hkv):
            for j in range(S // QBLOCK):
                dqu, tokens, dku, dvu = _unit_grads(q, k_cache, v_cache, d_o, t_hist,
                                                    group_idx[b, kvh, j], b, kvh, j, scale, group_size)
                h0 = kvh * group_size
                dq[b, h0:h0 + group_size, j * QBLOCK:(j + 1) * QBLOCK] = dqu.reshape(group_size, QBLOCK, d)
                act = tokens >= t_hist                       # history gets nothing (R-grad)
                np.add.at(dk[b, kvh], tokens[act] - t_hist, dku[act])
                np.add.at(dv[b, kvh], tokens[act] - t_hist, dvu[act])
    return dq, dk, dv


def dq_unit(q, k_cache, v_cache, d_o, t_hist, group_sel, b, kvh, j, scale, group_size):
    """dQ rows of one unit, [G*64, d] float64 (for sampled comparisons)."""
    return _unit_grads(q, k_cache, v_cache, d_o, t_hist, group_sel, b, kvh, j, scale, group_size)[0]


def dkdv_active_chunk(q, k_cache, v_cache, d_o, t_hist, group_idx, b, kvh, cc, scale, group_size):
    """dK, dV [64, d] of active chunk cc (tokens t_hist + 64cc ...) summed over every
    block that attends it: its own block (causally) and each later block that
    selected one of its groups."""
    S = q.shape[2]
    d = q.shape[3]
    lo = t_hist + cc * CHUNK
    dk = np.zeros((CHUNK, d))
    dv = np.zeros((CHUNK, d))
    for j in range(cc, S // QBLOCK):
        sel = group_idx[b, kvh, j]
        if j != cc and not np.any((sel >= lo // GROUP) & (sel < (lo + CHUNK) // GROUP)):
            continue
        _, tokens, dku, dvu = _unit_grads(q, k_cache, v_cache, d_o, t_hist, sel, b, kvh, j,
                                          scale, group_size)
        m = (tokens >= lo) & (tokens < lo + CHUNK)
        np.add.at(dk, tokens[m] - lo, dku[m])
        np.add.at(dv, tokens[m] - lo, dvu[m])
    return dk, dv


# ---------------------------------------------------------------------------
# Generation: one new token per sequence (reading R-decode).  HGA can be used
# for generation (adnankhan.ai note, "Raw Abstract / Excerpt"; seventnews,
# "检索：密集基线无退化"); the pages give no design for it.
# ---------------------------------------------------------------------------

def decode_route_unit(q_tok, chunk_sum, group_sum, pos, b, kvh, top_chunks, top_groups, group_size):
    """Routing of the token at position pos of sequence b for KV head kvh.
    q_tok [B, Hq, d]: the new tokens' queries.  Returns route_rows' tuple."""
    J = pos // CHUNK
    h0 = kvh * group_size
    rows = q_tok[b, h0:h0 + group_size].astype(np.float64)          # [G, d]
    return route_rows(rows, chunk_sum, group_sum, J, b, kvh, top_chunks, top_groups)


def decode_route(q_tok, chunk_sum, group_sum, pos, top_chunks, top_groups, group_size):
    """chunk_idx [B, Hkv, k_c], group_idx [B, Hkv, k_g] (int32, ascending, -1 padded)
    and the per-unit score tables; pos [B] (negative: idle slot)."""
    B, Hkv = chunk_sum.shape[:2]
    cidx = np.full((B, Hkv, top_chunks), -1, np.int32)
    gidx = np.full((B, Hkv, top_groups), -1, np.int32)
    tables = {}
    for b in range(B):
        if pos[b] < 0:
            continue
        for kvh in range(Hkv):
            cs, gs, sig, gids, tau = decode_route_unit(q_tok, chunk_sum, group_sum, int(pos[b]), b, kvh,
                                                       top_chunks, top_groups, group_size)
            cidx[b, kvh, :len(cs)] = cs
            gidx[b, kvh, :len(gs)] = gs
            tables[(b, kvh)] = (sig, gids, tau)
    return cidx, gidx, tables


def decode_key_tokens(group_sel, pos):
    """Positions the token at pos attends: the selected groups' tokens, then its own
    chunk up to and including itself."""
    J = pos // CHUNK
    return np.concatenate([key_tokens(group_sel), np.arange(J * CHUNK, pos + 1)])


def decode_attend(q_tok, k_cache, v_cache, pos, group_idx, scale, group_size):
    """O [B, Hq, d] and LSE [B, Hq] (float64) of the new tokens."""
    B, Hq, d = q_tok.shape
    Hkv = k_cache.shape[1]
    o = np.zeros((B, Hq, d), np.float64)
    lse = np.full((B, Hq), -np.inf, np.float64)
    for b in range(B):
        if pos[b] < 0:
            continue
        for kvh in range(Hkv):
            tok = decode_key_tokens(group_idx[b, kvh], int(pos[b]))
            keys = k_cache[b, kvh][tok].astype(np.float64)
            vals = v_cache[b, kvh][tok].astype(np.float64)
            h0 = kvh * group_size
            rows = q_tok[b, h0:h0 + group_size].astype(np.float64)
            L = scale * (rows @ keys.T)
            m = L.max(axis=1, keepdims=True)
            lu = m[:, 0] + np.log(np.exp(L - m).sum(axis=1))
            o[b, h0:h0 + group_size] = np.exp(L - lu[:, None]) @ vals
            lse[b, h0:h0 + group_size] = lu
    return o, lse


def decode_summaries(k_cache, pos, dtype, group_sum, chunk_sum):
    """Incremental summary update: for every sequence whose new token completes a
    chunk ((pos + 1) % 64 == 0), build that chunk's group and chunk summaries."""
    for b in range(k_cache.shape[0]):
        p = int(pos[b])
        if p >= 0 and (p + 1) % CHUNK == 0:
            c0 = p + 1 - CHUNK
            build_summaries(k_cache[b:b + 1], c0, c0 + CHUNK, dtype, group_sum[b:b + 1], chunk_sum[b:b + 1])
