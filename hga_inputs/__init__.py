"""Seeded synthetic workloads for the HGA routed-attention layer.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic: both the CPU oracle (through the
tests) and the GPU path consume exactly the arrays produced here.

Shapes follow the Qwen3-8B attention layout used on the pages (32 query heads,
8 KV heads, head_dim 128) with 2,048-token segments (segment-wise backprop,
"Long-Context Fine-Tuning with Limited VRAM", abstract and the HGA section of
the seventnews article), 64-token chunks and 8-token groups (same HGA section).

Layouts (row-major, contiguous):
  q, do           [B, Hq, S, d]
  k_cache, v_cache[B, Hkv, t_cap, d]   history at [0, t_hist), active segment
                                       at [t_hist, t_hist + S)
Float tensors are returned as float32 arrays whose values are exactly
representable in the workload dtype (bf16-rounded with round-to-nearest-even
for bf16 workloads), plus helpers to get the raw bf16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

CHUNK = 64
GROUP = 8
QBLOCK = 64


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact (as int16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-exact; call round_to_bf16 first")
    return (u >> 16).astype(np.uint16).view(np.int16)


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    t_hist: int
    seg_len: int
    t_cap: int
    top_chunks: int
    top_groups: int
    dtype: str                    # "f32" or "bf16"
    softmax_scale: float
    backward: bool
    q: np.ndarray                 # [B,Hq,S,d] float32 (dtype-exact)
    k_cache: np.ndarray           # [B,Hkv,t_cap,d]
    v_cache: np.ndarray           # [B,Hkv,t_cap,d]
    d_o: Optional[np.ndarray]     # [B,Hq,S,d] or None
    extra: Dict[str, object] = dataclasses.field(default_factory=dict)

    @property
    def group_size(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _cast(x, dtype):
    return round_to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def random_layer(*, seed: int, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 t_hist: int, seg_len: int, t_cap: Optional[int] = None, top_chunks: int,
                 top_groups: int, dtype: str = "bf16", backward: bool = True,
                 chunk_mean_var: float = 0.0, softmax_scale: Optional[float] = None,
                 name: str = "random") -> Workload:
    """Q, K, V, dO ~ N(0, 1); optionally K += a per-(sequence, KV head, chunk)
    mean drawn from N(0, chunk_mean_var * I) (block-structured keys)."""
    t_cap = t_hist + seg_len if t_cap is None else t_cap
    t = t_hist + seg_len
    rq, rk, rv, rdo, rs = _streams(seed, 5)
    q = _normal(rq, (batch, n_q_heads, seg_len, head_dim))
    k = np.zeros((batch, n_kv_heads, t_cap, head_dim), np.float32)
    v = np.zeros((batch, n_kv_heads, t_cap, head_dim), np.float32)
    k[:, :, :t] = _normal(rk, (batch, n_kv_heads, t, head_dim))
    v[:, :, :t] = _normal(rv, (batch, n_kv_heads, t, head_dim))
    if chunk_mean_var > 0.0:
        nch = t // CHUNK
        mu = _normal(rs, (batch, n_kv_heads, nch, head_dim)) * np.float32(math.sqrt(chunk_mean_var))
        k[:, :, :t] += np.repeat(mu, CHUNK, axis=2)
    d_o = _normal(rdo, (batch, n_q_heads, seg_len, head_dim)) if backward else None
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale
    return Workload(name=name, batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                    head_dim=head_dim, t_hist=t_hist, seg_len=seg_len, t_cap=t_cap,
                    top_chunks=top_chunks, top_groups=top_groups, dtype=dtype,
                    softmax_scale=scale, backward=backward, q=_cast(q, dtype),
                    k_cache=_cast(k, dtype), v_cache=_cast(v, dtype),
                    d_o=None if d_o is None else _cast(d_o, dtype))


def prev_query_block(*, seed: int, batch: int, n_q_heads: int, head_dim: int,
                     dtype: str = "bf16") -> np.ndarray:
    """Queries of the last 64-token block of the previous segment, [B, Hq, 64, d],
    N(0, 1) (the rows that route a segment's first block under causal routing)."""
    (r,) = _streams(seed + 7000, 1)
    return _cast(_normal(r, (batch, n_q_heads, QBLOCK, head_dim)), dtype)


@dataclasses.dataclass
class DecodeWorkload:
    """One generation step: every sequence adds one token at its own position."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    t_cap: int
    top_chunks: int
    top_groups: int
    dtype: str
    softmax_scale: float
    pos: np.ndarray               # [B] int64: the new token's position (negative: idle slot)
    q: np.ndarray                 # [B,Hq,d] the new tokens' queries
    k_cache: np.ndarray           # [B,Hkv,t_cap,d] (holds the new tokens' keys at pos)
    v_cache: np.ndarray

    @property
    def group_size(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def decode_batch(*, seed: int, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, t_cap: int,
                 pos, top_chunks: int, top_groups: int, dtype: str = "bf16", chunk_mean_var: float = 0.0,
                 name: str = "decode") -> DecodeWorkload:
    """Q, K, V ~ N(0, 1) over the whole cache (positions after a sequence's pos are
    filled too: they must not matter); optional per-(sequence, KV head, chunk) key
    means ~ N(0, chunk_mean_var * I)."""
    rq, rk, rv, rs = _streams(seed, 4)
    q = _normal(rq, (batch, n_q_heads, head_dim))
    k = _normal(rk, (batch, n_kv_heads, t_cap, head_dim))
    v = _normal(rv, (batch, n_kv_heads, t_cap, head_dim))
    if chunk_mean_var > 0.0:
        mu = _normal(rs, (batch, n_kv_heads, t_cap // CHUNK, head_dim)) * np.float32(math.sqrt(chunk_mean_var))
        k += np.repeat(mu, CHUNK, axis=2)
    return DecodeWorkload(name=name, batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                          head_dim=head_dim, t_cap=t_cap, top_chunks=top_chunks, top_groups=top_groups,
                          dtype=dtype, softmax_scale=1.0 / math.sqrt(head_dim),
                          pos=np.asarray(pos, np.int64), q=_cast(q, dtype), k_cache=_cast(k, dtype),
                          v_cache=_cast(v, dtype))


def decode_b8_ctx32k(seed: int = 66) -> DecodeWorkload:
    """Generation at 32K context: 8 sequences of the Qwen3-8B layer shape, each adding
    one token at a position in the last chunk of the 32,768-token cache (ragged
    own-chunk lengths, the last one completes its chunk), block-structured keys."""
    pos = [32767 - 9 * b for b in range(8)]
    return decode_batch(seed=seed, batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, t_cap=32768, pos=pos,
                        top_chunks=16, top_groups=64, chunk_mean_var=0.5, name="decode_b8_ctx32k")


def decode_b64_ctx16k(seed: int = 67) -> DecodeWorkload:
    """Generation at serving batch size: 64 sequences of the Qwen3-8B layer shape at
    16K context, each adding one token in the last chunks of its 16,384-token cache
    (ragged own-chunk lengths; every 64th position completes a chunk), block-structured
    keys.  Timing only: at 8 sequences the generation kernels cannot fill the chip."""
    pos = [16383 - 9 * b for b in range(64)]
    return decode_batch(seed=seed, batch=64, n_q_heads=32, n_kv_heads=8, head_dim=128, t_cap=16384, pos=pos,
                        top_chunks=16, top_groups=64, chunk_mean_var=0.5, name="decode_b64_ctx16k")


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

def tiny_f32(full_coverage: bool = False) -> Workload:
    """1 sequence, 1 head, head_dim 64, one 1,024-token segment, fp32, fwd only;
    top-4 chunks / top-8 groups (or the full-coverage budget 16 / 128)."""
    kc, kg = (16, 128) if full_coverage else (4, 8)
    return random_layer(seed=11, batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64, t_hist=0,
                        seg_len=1024, top_chunks=kc, top_groups=kg, dtype="f32",
                        backward=False, name="tiny_f32_1k" + ("_full" if full_coverage else ""))


def qwen_2k_hist() -> Workload:
    """Qwen3-8B-shaped layer, 2,048 active + 2,048 history tokens, bf16, fwd+bwd."""
    return random_layer(seed=22, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                        t_hist=2048, seg_len=2048, top_chunks=16, top_groups=64,
                        name="qwen3_8b_layer_ctx4k")


def qwen_16k() -> Workload:
    """Qwen3-8B-shaped layer at 16,384 context (14,336 history + 2,048 active),
    block-structured keys (per-chunk mean ~ N(0, 0.5 I) plus N(0, I) noise)."""
    return random_layer(seed=33, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                        t_hist=14336, seg_len=2048, top_chunks=16, top_groups=64,
                        chunk_mean_var=0.5, name="qwen3_8b_layer_ctx16k")


def rollout_segment(s: int, *, n_q_heads=32, n_kv_heads=8, head_dim=128, seg_len=2048,
                    seed: int = 44, n_segments: int = 64):
    """Segment s of the 131,072-token evaluation rollout: Q, K, V of that segment
    (block-structured keys), bf16. Returns (q [1,Hq,S,d], k [1,Hkv,S,d], v [1,Hkv,S,d])."""
    ss = np.random.SeedSequence(seed).spawn(n_segments)[s]
    rq, rk, rv, rs = [np.random.Generator(np.random.PCG64(x)) for x in ss.spawn(4)]
    q = _normal(rq, (1, n_q_heads, seg_len, head_dim))
    k = _normal(rk, (1, n_kv_heads, seg_len, head_dim))
    v = _normal(rv, (1, n_kv_heads, seg_len, head_dim))
    mu = _normal(rs, (1, n_kv_heads, seg_len // CHUNK, head_dim)) * np.float32(math.sqrt(0.5))
    k += np.repeat(mu, CHUNK, axis=2)
    return round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)


ROLLOUT_TOKENS = 131072
ROLLOUT_SEG = 2048


def planted_batch(batch: int = 8, t_total: int = 32768, seg_len: int = 2048,
                  n_q_heads: int = 32, n_kv_heads: int = 8, head_dim: int = 128,
                  n_planted: int = 4, cos: float = 0.9, q_plant: float = 1.0,
                  seed: int = 55, top_chunks: int = 16, top_groups: int = 64,
                  n_decoys: int = 0) -> Workload:
    """batch x 32,768-token sequences; fwd+bwd of the last 2,048-token segment.
    Per sequence: a random unit direction u; n_planted distinct history chunks
    whose keys (every KV head, every token) have cosine `cos` with u at their
    own norm; every query of the active segment gets + q_plant * u.  With
    n_decoys > 0, that many further distinct chunks get cosine -cos with u (a
    control for direction sensitivity: their summaries are as large as the
    planted ones but point away from the queries)."""
    t_hist = t_total - seg_len
    w = random_layer(seed=seed, batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                     head_dim=head_dim, t_hist=t_hist, seg_len=seg_len, top_chunks=top_chunks,
                     top_groups=top_groups, dtype="f32", name="planted")
    rp = _streams(seed + 1000, batch)
    planted = np.zeros((batch, n_planted), np.int64)
    decoys = np.zeros((batch, n_decoys), np.int64)
    q = w.q
    k = w.k_cache
    for b in range(batch):
        u = _normal(rp[b], (head_dim,)).astype(np.float64)
        u /= np.linalg.norm(u)
        picks = rp[b].choice(t_hist // CHUNK, size=n_planted + n_decoys, replace=False)
        planted[b] = np.sort(picks[:n_planted])
        decoys[b] = np.sort(picks[n_planted:])
        for c, cs in [(c, cos) for c in planted[b]] + [(c, -cos) for c in decoys[b]]:
            g = k[b, :, c * CHUNK:(c + 1) * CHUNK].astype(np.float64)       # [Hkv,64,d]
            gn = np.linalg.norm(g, axis=-1, keepdims=True)
            wperp = g - (g @ u)[..., None] * u
            wperp /= np.linalg.norm(wperp, axis=-1, keepdims=True)
            k[b, :, c * CHUNK:(c + 1) * CHUNK] = (gn * (cs * u + math.sqrt(1 - cs * cs) * wperp)).astype(np.float32)
        q[b] = (q[b].astype(np.float64) + q_plant * u).astype(np.float32)
    return Workload(name=f"planted_b{batch}_ctx{t_total}", batch=batch, n_q_heads=n_q_heads,
                    n_kv_heads=n_kv_heads, head_dim=head_dim, t_hist=t_hist, seg_len=seg_len,
                    t_cap=t_total, top_chunks=top_chunks, top_groups=top_groups, dtype="bf16",
                    softmax_scale=1.0 / math.sqrt(head_dim), backward=True,
                    q=round_to_bf16(q), k_cache=round_to_bf16(k), v_cache=round_to_bf16(w.v_cache),
                    d_o=round_to_bf16(w.d_o), extra={"planted_chunks": planted, "decoy_chunks": decoys})


NAMED = {
    "tiny_f32_1k": tiny_f32,
    "qwen3_8b_layer_ctx4k": qwen_2k_hist,
    "qwen3_8b_layer_ctx16k": qwen_16k,
    "planted_b8_ctx32k": planted_batch,
}
