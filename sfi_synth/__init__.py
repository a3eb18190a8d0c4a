"""Seeded synthetic inputs for the Slow-Fast Inference (SFI) decode-attention path.

This module is shared by the tests, the bench and ``smoke()``.  It only draws
numbers and lays them out the way the library expects them (paged K/V pools,
random-permutation block tables, planted heavy-hitter keys, per-request
lengths).  It computes none of the method's arithmetic: no logits, no softmax,
no selection, no packing.

Workload shapes follow the SFI page (thelatestinai.com/papers/2603.12038,
Fig. 2: a managed sparse state of sink + selected + recent tokens; Fig. 3B:
recent tokens read in place from paged KV; Table 1: kernel-level speedups at
KV length 16K in bf16).

Draw order inside one case is fixed: per-request lengths (if random), the
block-table permutation, Q, the K pool, the V pool, heavy-hitter positions,
extra query steps.  Every generator is ``numpy.random.Generator(PCG64(seed))``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

PAGE_SIZE = 16

__all__ = [
    "PAGE_SIZE", "bf16_bits", "bf16_values", "PagedKV", "Case",
    "make_case", "tiny_case", "qwen06b_decode_case", "qwen8b_batched_case",
    "refresh64k_case", "specmix128k_case", "retention_budget", "RETENTIONS", "DriftCase", "drifting_case",
]


# --------------------------------------------------------------------------- bf16 storage

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """The exact float32 values held by raw bfloat16 bits."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")


def _values(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_values(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def _draw_pool(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    """N(0, 1) values in storage form, drawn in order in chunks (the same stream as one
    draw of the whole array) so that large pools never exist as float32."""
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    flat = out.reshape(-1)
    for i in range(0, flat.size, chunk):
        n = min(chunk, flat.size - i)
        flat[i:i + n] = _store(rng.standard_normal(n, dtype=np.float32), dtype)
    return out


# --------------------------------------------------------------------------- containers

@dataclass
class PagedKV:
    """A paged K/V pool.

    ``k`` and ``v`` are storage arrays of shape ``[num_pages, Hkv, page_size, d]``
    (uint16 bf16 bits or float32).  Token ``j`` of request ``b`` for KV head ``g``
    lives at ``[block_table[b, j // page_size], g, j % page_size, :]``.
    Unused block-table entries hold -1.
    """
    dtype: str
    k: np.ndarray
    v: np.ndarray
    block_table: np.ndarray
    page_size: int = PAGE_SIZE

    @property
    def num_pages(self) -> int:
        return int(self.k.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def k_values(self) -> np.ndarray:
        return _values(self.k, self.dtype)

    def v_values(self) -> np.ndarray:
        return _values(self.v, self.dtype)

    def slot(self, b: int, pos: int) -> Tuple[int, int]:
        return int(self.block_table[b, pos // self.page_size]), pos % self.page_size


@dataclass
class Case:
    """One synthetic decode-attention workload.

    ``q`` has shape ``[B, t_q, Hq, d]`` (storage dtype as the pool).  ``seq_lens[b]``
    counts every token of request b including its ``t_q`` query tokens, whose K/V
    are already in the pool.  ``extra_q`` holds further query steps (for fast
    steps after a slow step), shape ``[steps, B, Hq, d]``.
    """
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    d: int
    t_q: int
    q: np.ndarray
    kv: PagedKV
    seq_lens: np.ndarray
    n_sink: int
    n_recent: int
    k_sel: int
    scale: float
    planted: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)
    extra_q: Optional[np.ndarray] = None
    modes: Optional[np.ndarray] = None       # per request: 0 = sparse draft, 1 = dense verify
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def q_values(self) -> np.ndarray:
        return _values(self.q, self.dtype)

    def extra_q_values(self) -> np.ndarray:
        return _values(self.extra_q, self.dtype)


# --------------------------------------------------------------------------- builders

def _block_table(rng: np.random.Generator, capacity: List[int], page_size: int,
                 spare_pages: int) -> Tuple[np.ndarray, int]:
    pages_per_req = [-(-c // page_size) for c in capacity]
    num_pages = int(sum(pages_per_req)) + spare_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = max(pages_per_req) if pages_per_req else 1
    bt = np.full((len(capacity), max(1, max_pages)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per_req):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, num_pages


def make_case(seed: int, *, name: str, B: int, Hq: int, Hkv: int, d: int, dtype: str,
              seq_lens, n_sink: int, n_recent: int, k_sel: int, t_q: int = 1,
              hh_per_head: int = 0, capacity=None, extra_steps: int = 0,
              extra_noise: float = 0.25, spare_pages: int = 0,
              scale: Optional[float] = None) -> Case:
    """Build a case with Q, K, V ~ N(0, 1) and optional planted heavy-hitter keys.

    Heavy hitters (the workload's "K aligned to Q, scaled x4"): for each (b, g),
    ``hh_per_head`` positions are drawn uniformly without replacement from
    ``[n_sink, seq_lens[b] - t_q + 1 - n_recent)`` and their keys are set to
    4 * (mean of the group's query vectors of the first query token).
    ``extra_steps`` further query steps are drawn as q0 + extra_noise * N(0, 1).
    ``capacity[b]`` (default ``seq_lens[b]``) sizes the pool for later appends.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    cap = [int(c) for c in (capacity if capacity is not None else seq_lens)]
    bt, num_pages = _block_table(rng, cap, PAGE_SIZE, spare_pages)
    G = Hq // Hkv
    q = rng.standard_normal((B, t_q, Hq, d), dtype=np.float32)
    k = _draw_pool(rng, (num_pages, Hkv, PAGE_SIZE, d), dtype)
    v = _draw_pool(rng, (num_pages, Hkv, PAGE_SIZE, d), dtype)
    q_st = _store(q, dtype)
    qv = _values(q_st, dtype)
    planted: Dict[Tuple[int, int], np.ndarray] = {}
    if hh_per_head > 0:
        for b in range(B):
            lo, hi = n_sink, int(seq_lens[b]) - t_q + 1 - n_recent
            n = min(hh_per_head, max(0, hi - lo))
            for g in range(Hkv):
                if n == 0:
                    continue
                pos = np.sort(rng.choice(hi - lo, size=n, replace=False) + lo).astype(np.int64)
                planted[(b, g)] = pos
                qbar = qv[b, 0, g * G:(g + 1) * G, :].astype(np.float64).mean(axis=0)
                key = _store((4.0 * qbar).astype(np.float32), dtype)
                k[bt[b, pos // PAGE_SIZE], g, pos % PAGE_SIZE, :] = key
    extra = None
    if extra_steps > 0:
        noise = rng.standard_normal((extra_steps, B, Hq, d), dtype=np.float32)
        extra = _store(qv[None, :, 0, :, :] + np.float32(extra_noise) * noise, dtype)
    kv = PagedKV(dtype=dtype, k=k, v=v, block_table=bt)
    return Case(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, d=d, t_q=t_q, q=q_st, kv=kv,
                seq_lens=seq_lens, n_sink=n_sink, n_recent=n_recent, k_sel=k_sel,
                scale=float(scale if scale is not None else 1.0 / np.sqrt(d)),
                planted=planted, extra_q=extra)


# Table 1 of the SFI page lists retention ratios 1.6 ... 100 %; as fractions of the
# KV length they are 1/64, 1/16, 1/8, 1/4, 3/8, 1/2, 3/4, 63/64 and 1.
RETENTIONS = [(1, 64), (1, 16), (1, 8), (1, 4), (3, 8), (1, 2), (3, 4), (63, 64), (1, 1)]


def retention_budget(L: int, frac: Tuple[int, int], n_sink: int, n_recent: int) -> int:
    """Selected budget k so that sink + selected + recent = L * frac tokens."""
    total = (L * frac[0]) // frac[1]
    return max(0, total - n_sink - n_recent)


def tiny_case(seed: int = 1) -> Case:
    """fp32, 1 request, 4 query heads on 1 KV head, d=64, KV length 1024 (pool for 1032),
    sink 4, selected 64, recent 32, 8 planted heavy hitters, 8 further query steps."""
    return make_case(seed, name="tiny_fp32", B=1, Hq=4, Hkv=1, d=64, dtype="f32",
                     seq_lens=[1024], capacity=[1032], n_sink=4, n_recent=32, k_sel=64,
                     hh_per_head=8, extra_steps=8, extra_noise=0.25)


def qwen06b_decode_case(seed: int = 2, L: int = 16384, B: int = 1,
                        frac: Tuple[int, int] = (1, 8)) -> Case:
    """bf16, 16 query heads / 8 KV heads, d=128, sink 4, recent 64, ~2 % planted heavy hitters."""
    n_sink, n_recent = 4, 64
    k = retention_budget(L, frac, n_sink, n_recent)
    c = make_case(seed, name=f"qwen06b_L{L}_B{B}", B=B, Hq=16, Hkv=8, d=128, dtype="bf16",
                  seq_lens=[L] * B, n_sink=n_sink, n_recent=n_recent, k_sel=k,
                  hh_per_head=max(1, round(0.02 * L)))
    c.meta["retention"] = frac
    return c


def qwen8b_batched_case(seed: int = 3, B: int = 16, lo: int = 16384, hi: int = 32768) -> Case:
    """bf16, 32 query heads / 8 KV heads, d=128, per-request lengths uniform in [lo, hi],
    sink 4, selected 1024, recent 256, 256 planted keys per (request, KV head)."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    return make_case(seed, name=f"qwen8b_B{B}", B=B, Hq=32, Hkv=8, d=128, dtype="bf16",
                     seq_lens=lens, n_sink=4, n_recent=256, k_sel=1024, hh_per_head=256)


def refresh64k_case(seed: int = 4, B: int = 4, L: int = 65536) -> Case:
    """bf16, 32 query heads / 8 KV heads, d=128, KV length 64K, sink 4, recent 256, top-2048."""
    return make_case(seed, name=f"refresh_L{L}_B{B}", B=B, Hq=32, Hkv=8, d=128, dtype="bf16",
                     seq_lens=[L] * B, n_sink=4, n_recent=256, k_sel=2048,
                     hh_per_head=max(1, round(0.02 * (L - 260))))


def specmix128k_case(seed: int = 5, B: int = 8, L: int = 131072, t_q: int = 8,
                     n_draft: Optional[int] = None) -> Case:
    """bf16, 32 query heads / 8 KV heads, d=128.  Requests [0, n_draft) draft sparsely
    (one query token, 5 % retention: sink 4 + recent 256 + selected), the rest verify
    ``t_q`` draft tokens densely.  Query tensor is laid out per request with ``t_q``
    rows; draft requests use row 0 only."""
    n_draft = B // 2 if n_draft is None else n_draft
    n_sink, n_recent = 4, 256
    budget = int(round(0.05 * L))
    c = make_case(seed, name=f"specmix_L{L}_B{B}", B=B, Hq=32, Hkv=8, d=128, dtype="bf16",
                  seq_lens=[L] * B, n_sink=n_sink, n_recent=n_recent,
                  k_sel=max(0, budget - n_sink - n_recent), t_q=t_q,
                  hh_per_head=max(1, round(0.02 * (L - t_q + 1 - n_sink - n_recent))))
    c.modes = np.array([0] * n_draft + [1] * (B - n_draft), dtype=np.int32)
    return c


# --------------------------------------------------------------------------- drifting support

@dataclass
class DriftCase:
    """A decode run whose heavy hitters persist for ``period`` query steps, then shift.

    ``case`` holds the pools (sized for every step's token) with ``seq_lens`` = L0, the
    lengths before the first step.  Step t decodes the token at position L0 + t, whose
    K/V already sit in the pool, so the request length at step t is L0 + t + 1.
    ``q_steps`` [steps, B, Hq, d] are the queries (storage form) and ``support``
    [epochs, B, Hkv, hh] the planted positions of each epoch (sorted)."""
    case: Case
    steps: int
    period: int
    q_steps: np.ndarray
    support: np.ndarray

    def q_step_values(self) -> np.ndarray:
        return _values(self.q_steps, self.case.dtype)


def drifting_case(seed: int, *, B: int, Hq: int, Hkv: int, d: int, dtype: str, L0, steps: int,
                  period: int, hh: int, n_sink: int, n_recent: int, k_sel: int,
                  noise: float = 0.25) -> DriftCase:
    """Heavy hitters that persist across ``period`` consecutive query steps, then shift.

    Epoch e = t // period has, per (request b, KV head g), a direction u ~ N(0, 1)^d and
    ``hh`` positions drawn without replacement from [n_sink, L0_b - n_recent) (disjoint
    from every other epoch's); their keys are set to 4 u.  The queries of step t are
    u_e(t),b,g(h) + noise * N(0, 1) for every query head h of group g.  Draw order: the
    pools (as make_case with no planting), then per epoch the directions and positions,
    then the query noise."""
    L0 = np.broadcast_to(np.asarray(L0, dtype=np.int32), (B,)).copy()
    c = make_case(seed, name="drift", B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, seq_lens=L0,
                  capacity=[int(x) + steps for x in L0], n_sink=n_sink, n_recent=n_recent, k_sel=k_sel)
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    G = Hq // Hkv
    E = (steps + period - 1) // period
    u = rng.standard_normal((E, B, Hkv, d), dtype=np.float32)
    support = np.zeros((E, B, Hkv, hh), dtype=np.int64)
    bt = c.kv.block_table
    for b in range(B):
        lo, hi = n_sink, int(L0[b]) - n_recent
        if hi - lo < E * hh:
            raise ValueError("not enough candidate positions for the planted support")
        for g in range(Hkv):
            pos = rng.choice(hi - lo, size=E * hh, replace=False) + lo
            for e in range(E):
                pe = np.sort(pos[e * hh:(e + 1) * hh]).astype(np.int64)
                support[e, b, g] = pe
                key = _store((4.0 * u[e, b, g]).astype(np.float32), dtype)
                c.kv.k[bt[b, pe // PAGE_SIZE], g, pe % PAGE_SIZE, :] = key
    eps = rng.standard_normal((steps, B, Hq, d), dtype=np.float32)
    epoch = np.arange(steps) // period
    dirs = u[epoch][:, :, np.repeat(np.arange(Hkv), G), :]          # [steps, B, Hq, d]
    q_steps = _store(dirs + np.float32(noise) * eps, dtype)
    return DriftCase(case=c, steps=steps, period=period, q_steps=q_steps, support=support)
