"""Refresh schedules of the sparse state, driven through the C ABI.

RefreshSchedule: fixed-interval refresh of one layer.

SFI page, Fig. 2 and its caption: decoding alternates slow steps (dense attention
whose masked logits refresh the selected memory through the Selector) with fast
steps (attention over sink + selected + recent).  The pages trigger slow steps at
sentence boundaries; this driver refreshes every ``interval`` steps, the plainest
schedule that exercises the same path.  Every step is library launches only:

    slow step:  sfi_dense_attn_with_stats (t_q = 1) -> sfi_select_topk -> sfi_pack_compact
    fast step:  sfi_sparse_decode_attn

The driver owns the buffers of the sparse state (logits, selection, compact K/V,
n_compact), the outputs and the workspaces, and marshals each call once: a step costs
its launches and nothing else on the host.  The caller owns the paged pools, the
block table and the query and length buffers, writing the step's query into ``q``
and its lengths into ``seq_lens`` before calling :meth:`step` (the length includes
the token being decoded, whose K/V must already be in the pool).
"""
from typing import Optional

import torch

from . import (bind, dense_attn_with_stats, pack_compact, select_topk, sparse_decode_attn,
               sparse_decode_indexed_attn, workspace_size)


class RefreshSchedule:
    """One layer's SFI state for a batch of requests, refreshed every ``interval`` steps."""

    def __init__(self, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                 q: torch.Tensor, seq_lens: torch.Tensor, *, max_seq_len: int, n_sink: int, n_recent: int,
                 k: int, interval: int, scale: Optional[float] = None, stream=None):
        if interval < 1:
            raise ValueError("interval must be >= 1")
        if q.dim() != 3:
            raise ValueError("q must be [B, Hq, d]")
        B, Hq, d = q.shape
        Hkv = k_pool.shape[1]
        dev = q.device
        self.interval = interval
        self.t = 0
        self.q, self.seq_lens = q, seq_lens
        self.cap = n_sink + k
        f32 = dict(dtype=torch.float32, device=dev)
        self.out = torch.empty((B, Hq, d), **f32)
        self.lse = torch.empty((B, Hq), **f32)
        self.scores = torch.empty((B, Hkv, max_seq_len), **f32)
        self.sel = torch.full((B, Hkv, k), -1, dtype=torch.int32, device=dev)
        self.compact_k = torch.zeros((B, Hkv, self.cap, d), dtype=k_pool.dtype, device=dev)
        self.compact_v = torch.zeros_like(self.compact_k)
        self.n_compact = torch.zeros((B,), dtype=torch.int32, device=dev)
        common = dict(k_pool=k_pool, block_table=block_table, Hq=Hq, dtype=k_pool.dtype, max_seq_len=max_seq_len)
        ws_d = torch.zeros(workspace_size("dense", **common) + 16, dtype=torch.uint8, device=dev)
        ws_s = torch.zeros(workspace_size("sparse", cap=self.cap, n_recent=n_recent, **common) + 16,
                           dtype=torch.uint8, device=dev)
        self._buffers = (ws_d, ws_s)
        q4 = q.view(B, 1, Hq, d)
        out4, lse3 = self.out.view(B, 1, Hq, d), self.lse.view(B, 1, Hq)
        self._slow = [
            bind(dense_attn_with_stats, q4, k_pool, v_pool, block_table, seq_lens, max_seq_len=max_seq_len,
                 n_sink=n_sink, n_recent=n_recent, scale=scale, out=out4, lse=lse3, scores=self.scores,
                 workspace=ws_d, stream=stream),
            bind(select_topk, self.scores, seq_lens, k=k, n_sink=n_sink, n_recent=n_recent, sel_idx=self.sel,
                 stream=stream),
            bind(pack_compact, k_pool, v_pool, block_table, seq_lens, self.sel, n_sink=n_sink, cap=self.cap,
                 max_seq_len=max_seq_len, compact_k=self.compact_k, compact_v=self.compact_v,
                 n_compact=self.n_compact, stream=stream),
        ]
        self._fast = bind(sparse_decode_attn, q, k_pool, v_pool, block_table, seq_lens, self.compact_k,
                          self.compact_v, self.n_compact, n_sink=n_sink, n_recent=n_recent,
                          max_seq_len=max_seq_len, scale=scale, out=self.out, lse=self.lse, workspace=ws_s,
                          stream=stream)

    def step(self) -> bool:
        """Decode one step into ``out`` / ``lse``; returns True when it was a slow step."""
        slow = self.t % self.interval == 0
        if slow:
            for call in self._slow:
                call()
        else:
            self._fast()
        self.t += 1
        return slow


class DraftRefresh:
    """Draft steps of a stack of layers with an intra-draft refresh layer.

    ASPIRE abstract (page 1): during drafting, one designated layer runs full attention
    and refreshes the sparse context at every draft step.  Reading: the designated
    layer's dense attention also yields the masked group logits, the Selector turns them
    into the selected set (per request and KV head), and every other layer attends over
    sink + that set + recent of its own K/V.  The set is shared, so the other layers
    read its rows in place through the block table (sfi_sparse_decode_indexed_attn)
    instead of packing a compact buffer per layer and step.  Layers before the
    designated one use the previous step's set, layers after it the new one.

    A step is, in layer order:  refresh layer: sfi_dense_attn_with_stats -> sfi_select_topk;
    every other layer: sfi_sparse_decode_indexed_attn.  All calls are marshalled once.

    The caller owns the pools (one (k_pool, v_pool) per layer, sharing the block table),
    the query buffer q [n_layers, B, Hq, d] and seq_lens, and writes the step's queries
    and lengths (which count the token being decoded, already in every pool) before
    calling step().  ``sel0`` [B, Hkv, k] is the set before the first step (default:
    empty, i.e. sink + recent only).
    """

    def __init__(self, pools, block_table: torch.Tensor, q: torch.Tensor, seq_lens: torch.Tensor, *,
                 max_seq_len: int, n_sink: int, n_recent: int, k: int, refresh_layer: int,
                 sel0: Optional[torch.Tensor] = None, scale: Optional[float] = None, stream=None):
        n_layers = len(pools)
        if not 0 <= refresh_layer < n_layers:
            raise ValueError("refresh_layer must index a layer")
        if q.dim() != 4 or q.shape[0] != n_layers:
            raise ValueError("q must be [n_layers, B, Hq, d]")
        _, B, Hq, d = q.shape
        k_pool0 = pools[0][0]
        Hkv = k_pool0.shape[1]
        dev = q.device
        f32 = dict(dtype=torch.float32, device=dev)
        self.out = torch.empty((n_layers, B, Hq, d), **f32)
        self.lse = torch.empty((n_layers, B, Hq), **f32)
        self.scores = torch.empty((B, Hkv, max_seq_len), **f32)
        self.sel = torch.full((B, Hkv, k), -1, dtype=torch.int32, device=dev)
        if sel0 is not None:
            self.sel.copy_(sel0)
        common = dict(k_pool=k_pool0, block_table=block_table, Hq=Hq, dtype=k_pool0.dtype, max_seq_len=max_seq_len)
        ws_d = torch.zeros(workspace_size("dense", **common) + 16, dtype=torch.uint8, device=dev)
        ws_s = torch.zeros(workspace_size("sparse", cap=n_sink + k, n_recent=n_recent, **common) + 16,
                           dtype=torch.uint8, device=dev)
        self._buffers = (ws_d, ws_s)
        self._calls = []
        for layer, (kp, vp) in enumerate(pools):
            ql = q[layer]
            if layer == refresh_layer:
                self._calls.append(bind(dense_attn_with_stats, ql.view(B, 1, Hq, d), kp, vp, block_table, seq_lens,
                                        max_seq_len=max_seq_len, n_sink=n_sink, n_recent=n_recent, scale=scale,
                                        out=self.out[layer].view(B, 1, Hq, d), lse=self.lse[layer].view(B, 1, Hq),
                                        scores=self.scores, workspace=ws_d, stream=stream))
                self._calls.append(bind(select_topk, self.scores, seq_lens, k=k, n_sink=n_sink, n_recent=n_recent,
                                        sel_idx=self.sel, stream=stream))
            else:
                self._calls.append(bind(sparse_decode_indexed_attn, ql, kp, vp, block_table, seq_lens, self.sel,
                                        n_sink=n_sink, n_recent=n_recent, max_seq_len=max_seq_len, scale=scale,
                                        out=self.out[layer], lse=self.lse[layer], workspace=ws_s, stream=stream))

    def step(self) -> None:
        """One draft step of every layer into ``out`` / ``lse`` (and the new set into ``sel``)."""
        for call in self._calls:
            call()
