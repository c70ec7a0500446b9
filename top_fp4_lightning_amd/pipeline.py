"""Composition of the C-ABI calls into the indexer's per-token steps.

Decode (one query per sequence), following the hierarchical indexer of "DeepSeek-V4.1 model
structure (3)" (blog.javazero.top, section "use shallow-layer scores to limit deep-layer
scoring"):
  1. idx_quantize_q         the Full layer's query
  2. idx_score_full         every visible key -> block-8 maxima (scores are not written)
  3. idx_build_pool         pin + top-2048 blocks -> candidate pool
  4. idx_score_pool_gather  the Full layer's own query over the pool, then idx_topk -> top-512.
     Exact: a top-512 key's block is outranked by at most 511 unpinned blocks, so it is in
     the pool, and a pooled key's score is computed by the same per-key arithmetic.
  5. for each Reindex layer: idx_quantize_q, idx_score_pool_gather, idx_topk -> its top-512.

Several queries per sequence (speculative verification of the draft positions, "DeepSeek-V4.1-Flash
inference-side full breakdown", section 8.2): the same decode step with group = positions per
sequence, so the Full scan reads each key once for all of them (the many-query scan).

Training form ("DeepSeek-V4.1 model structure (3)", sections "three details of the pool in the
code" and "the pool also acts in training"): every layer scores every visible position, and a
Reindex layer sets the scores outside the pool to -inf before its top-512. MaskFormPlan runs it for
all layers at once (the queries of every layer present together): one scan of the key cache
serves every layer's query, then the pool and one top-512 per row over the pooled positions
(idx_topk_pool; or the literal in-place mask and a top-512 over whole rows).

Prefill (a chunk of queries sharing one key range, causal): idx_score_full writes block maxima
for every query; idx_top_blocks keeps the 512 best blocks per query (a top-512 key's block is among
them); idx_score_pool_gather re-scores those 4096 keys; idx_topk takes the final 512.

All buffers are allocated once in the plan objects, so a step allocates nothing and can be
captured in a HIP graph.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (BLOCK, IDX_OP_BUILD_POOL, IDX_OP_TOPK, Recorded, idx_build_pool, idx_mask_pool, idx_quantize_q,
               idx_score_full, idx_score_pool_gather, idx_top_blocks, idx_topk, idx_topk_pool, record, workspace)


@dataclass
class DeviceWorkload:
    """Inputs resident in HBM: quantised key cache, raw bf16 queries per layer, fp32 weights."""

    signs: torch.Tensor  # int8 [128]
    k_codes: torch.Tensor  # u8 [N, 64]
    k_scales: torch.Tensor  # u8 [N, 4]
    k_base: torch.Tensor  # int64 [nq]
    n_vis: torch.Tensor  # int32 [nq]
    max_n: int
    group: int
    q: list  # per layer: bf16 [nq, 32, 128]
    w: list  # per layer: f32 [nq, 32]

    @property
    def nq(self) -> int:
        return int(self.n_vis.shape[0])

    @staticmethod
    def from_workload(wl, device="cuda", chunk_rows: int = 1 << 20, group: int | None = None) -> "DeviceWorkload":
        """Generate a seeded workload's keys on the host in chunks and quantise them on the GPU.
        `group` (default: the workload's) is the run of consecutive queries sharing a key range."""
        group = wl.group if group is None else group
        signs = torch.from_numpy(wl.signs()).to(device)
        total = wl.total_keys
        k_codes = torch.empty(total, 64, dtype=torch.uint8, device=device)
        k_scales = torch.empty(total, 4, dtype=torch.uint8, device=device)
        base = wl.seq_base
        for b in range(wl.nseq):
            n = int(wl.seq_len[b])
            for s0 in range(0, n, chunk_rows):
                cnt = min(chunk_rows, n - s0)
                raw = torch.from_numpy(wl.keys(b, s0, cnt).view(np.int16)).view(torch.bfloat16).to(device)
                r0 = int(base[b]) + s0
                idx_quantize_q(raw, signs, k_codes[r0:r0 + cnt], k_scales[r0:r0 + cnt])
        q = []
        w = []
        for layer in range(wl.layers + 1):
            qh = wl.q(layer)
            q.append(torch.from_numpy(qh.view(np.int16)).view(torch.bfloat16).to(device).contiguous())
            w.append(torch.from_numpy(wl.w(layer)).to(device).contiguous())
        return DeviceWorkload(signs=signs, k_codes=k_codes, k_scales=k_scales,
                              k_base=torch.from_numpy(wl.k_base).to(device),
                              n_vis=torch.from_numpy(wl.n_vis.astype(np.int32)).to(device),
                              max_n=int(wl.n_vis.max()) if wl.nq else 0, group=group, q=q, w=w)


class DecodePlan:
    """Preallocated buffers for one decode step (Full layer + pool + Reindex layers)."""

    def __init__(self, dev: DeviceWorkload, k: int = 512, topk_blocks: int = 2048, want_scores: bool = False):
        nq, max_n = dev.nq, dev.max_n
        d = dev.k_codes.device
        self.dev, self.k, self.topk_blocks = dev, k, topk_blocks
        self.layers = len(dev.q) - 1
        nb = (max_n + BLOCK - 1) // BLOCK
        self.max_blocks = min(topk_blocks, nb)
        slots = self.max_blocks * BLOCK
        self.q_codes = [torch.empty(nq, 32, 64, dtype=torch.uint8, device=d) for _ in dev.q]
        self.q_scales = [torch.empty(nq, 32, 4, dtype=torch.uint8, device=d) for _ in dev.q]
        self.block_max = torch.empty(nq, max(nb, 1), dtype=torch.float32, device=d)
        self.scores = torch.empty(nq, max(max_n, 1), dtype=torch.float32, device=d) if want_scores else None
        self.pool_blocks = torch.empty(nq, topk_blocks, dtype=torch.int32, device=d)
        self.pool_count = torch.empty(nq, dtype=torch.int32, device=d)
        self.pool_scores = [torch.empty(nq, max(slots, 1), dtype=torch.float32, device=d) for _ in dev.q]
        self.topk = [torch.empty(nq, k, dtype=torch.int32, device=d) for _ in dev.q]
        self.topk_val = [torch.empty(nq, k, dtype=torch.float32, device=d) for _ in dev.q]
        self.ws_pool = workspace(IDX_OP_BUILD_POOL, nq, max_n, topk_blocks, device=d)
        self.ws_topk = workspace(IDX_OP_TOPK, nq, max(slots, 1), k, device=d)

    def quantize(self, layer: int, stream=None):
        idx_quantize_q(self.dev.q[layer], self.dev.signs, self.q_codes[layer], self.q_scales[layer], stream=stream)

    def full_scan(self, stream=None):
        dv = self.dev
        idx_score_full(dv.k_codes, dv.k_scales, dv.k_base, dv.n_vis, self.q_codes[0], self.q_scales[0], dv.w[0],
                       dv.max_n, group=dv.group, scores=self.scores, block_max=self.block_max, stream=stream)

    def build_pool(self, stream=None):
        idx_build_pool(self.block_max, self.dev.n_vis, self.dev.max_n, self.pool_blocks, self.pool_count,
                       self.ws_pool, topk_blocks=self.topk_blocks, stream=stream)

    def pool_gather(self, layer: int, stream=None):
        dv = self.dev
        idx_score_pool_gather(dv.k_codes, dv.k_scales, dv.k_base, dv.n_vis, self.pool_blocks, self.pool_count,
                              self.max_blocks, self.q_codes[layer], self.q_scales[layer], dv.w[layer],
                              self.pool_scores[layer], stream=stream)

    def pool_select(self, layer: int, stream=None, events=None):
        if events is not None:
            events[0].record(stream)
        self.pool_gather(layer, stream)
        if events is not None:
            events[1].record(stream)
        idx_topk(self.pool_scores[layer], self.max_blocks * BLOCK, self.k, self.topk[layer], self.ws_topk,
                 out_val=self.topk_val[layer], blocks=self.pool_blocks, stream=stream)

    def run(self, stream=None):
        self.quantize(0, stream)
        self.full_scan(stream)
        self.build_pool(stream)
        self.pool_select(0, stream)
        for layer in range(1, self.layers + 1):
            self.quantize(layer, stream)
            self.pool_select(layer, stream)
        return self

    def compiled(self, stream=None) -> Recorded:
        """The step of run() recorded once: replaying it issues the same launches on the same
        stream without marshalling each call again on the host."""
        with record() as calls:
            self.run(stream)
        return Recorded(calls)


class TokenPlan:
    """The indexer work of one decode token across the model ("DeepSeek-V4.1 model structure
    (3)", the per-token table of section "Reindex layers score a million entries per token", and
    section "it is only in the decoder"): each encoder Full layer scans its own key cache and keeps
    its own top-512 (no pool in the encoder; the plan reaches the exact top-512 through block maxima
    and a gather, as for the decoder's Full layer), then the decoder's Full layer, pool and Reindex
    layers."""

    def __init__(self, encoders: list, decoder: DeviceWorkload, k: int = 512):
        self.encoders = [DecodePlan(d, k=k) for d in encoders]
        self.decoder = DecodePlan(decoder, k=k)

    def run(self, stream=None):
        for p in self.encoders:
            p.run(stream)
        self.decoder.run(stream)
        return self

    def compiled(self, stream=None) -> Recorded:
        """The token of run() recorded once (as DecodePlan.compiled)."""
        with record() as calls:
            self.run(stream)
        return Recorded(calls)


def decode_step(dev: DeviceWorkload, plan: DecodePlan | None = None, **kw) -> dict:
    plan = plan or DecodePlan(dev, **kw)
    plan.run()
    return {"topk": plan.topk[0], "topk_val": plan.topk_val[0], "pool_blocks": plan.pool_blocks,
            "pool_count": plan.pool_count, "block_max": plan.block_max,
            "reindex_topk": plan.topk[1:], "plan": plan}


class MaskFormPlan:
    """The decode step in its training form, all layers batched. Rows are stacked query-major
    (row = query * L + layer, L = Full layer + Reindex layers), so the rows of one key range stay
    consecutive and one many-query scan computes every layer's full score row (and the block
    maxima the Full layer's pool is built from). The mask then applies each query's pool to all
    of its rows. On the Full layer's row it changes no top-512 entry: a key outside the pool is
    outranked by a key of each of the 2047 unpinned pooled blocks (their maxima beat or tie-win
    its block's), so it never makes the top-512. The results equal DecodePlan's gather form.

    By default the mask and the top-512 are one call, idx_topk_pool, which reads each row only at
    its query's pooled positions and leaves the scores unmasked. write_mask=True runs the literal
    form instead: idx_mask_pool writes -inf outside the pool in place, then idx_topk selects over
    whole rows (for callers that consume the masked scores)."""

    def __init__(self, dev: DeviceWorkload, k: int = 512, topk_blocks: int = 2048, write_mask: bool = False):
        nq, max_n = dev.nq, dev.max_n
        d = dev.k_codes.device
        self.dev, self.k, self.topk_blocks, self.write_mask = dev, k, topk_blocks, write_mask
        self.max_blocks = min(topk_blocks, (max_n + BLOCK - 1) // BLOCK)
        self.L = L = len(dev.q)
        self.rows = rows = nq * L
        nb = (max_n + BLOCK - 1) // BLOCK
        self.q = torch.stack(dev.q, 1).reshape(rows, 32, 128).contiguous()
        self.w = torch.stack(dev.w, 1).reshape(rows, 32).contiguous()
        self.k_base = dev.k_base.repeat_interleave(L)
        self.n_vis = dev.n_vis.repeat_interleave(L)
        self.q_codes = torch.empty(rows, 32, 64, dtype=torch.uint8, device=d)
        self.q_scales = torch.empty(rows, 32, 4, dtype=torch.uint8, device=d)
        self.scores = torch.empty(rows, max(max_n, 1), dtype=torch.float32, device=d)
        self.block_max = torch.empty(rows, max(nb, 1), dtype=torch.float32, device=d)
        self.pool_blocks = torch.empty(nq, topk_blocks, dtype=torch.int32, device=d)
        self.pool_count = torch.empty(nq, dtype=torch.int32, device=d)
        self.topk = torch.empty(rows, k, dtype=torch.int32, device=d)
        self.topk_val = torch.empty(rows, k, dtype=torch.float32, device=d)
        self.ws_pool = workspace(IDX_OP_BUILD_POOL, nq, max_n, topk_blocks, device=d)
        self.ws_topk = workspace(IDX_OP_TOPK, rows, max(max_n, 1), k, device=d) if write_mask else None

    def layer_topk(self, layer: int):
        """(indices, values) [nq, k] of one layer."""
        return self.topk.view(-1, self.L, self.k)[:, layer], self.topk_val.view(-1, self.L, self.k)[:, layer]

    def run(self, stream=None, events=None):
        dv, L = self.dev, self.L
        idx_quantize_q(self.q, dv.signs, self.q_codes, self.q_scales, stream=stream)
        if events is not None:
            events[0].record()
        idx_score_full(dv.k_codes, dv.k_scales, self.k_base, self.n_vis, self.q_codes, self.q_scales, self.w,
                       dv.max_n, group=dv.group * L, scores=self.scores, block_max=self.block_max, stream=stream)
        if events is not None:
            events[1].record()
        full_bm = self.block_max.view(dv.nq, L, -1)[:, 0]  # the Full layer's rows
        idx_build_pool(full_bm, dv.n_vis, dv.max_n, self.pool_blocks, self.pool_count, self.ws_pool,
                       topk_blocks=self.topk_blocks, stream=stream)
        if self.write_mask:
            idx_mask_pool(self.scores, self.n_vis, dv.max_n, self.pool_blocks, self.pool_count, group=L,
                          stream=stream)
            idx_topk(self.scores, dv.max_n, self.k, self.topk, self.ws_topk, n_valid=self.n_vis,
                     out_val=self.topk_val, stream=stream)
        else:
            idx_topk_pool(self.scores, self.n_vis, dv.max_n, self.pool_blocks, self.pool_count, self.max_blocks,
                          self.k, self.topk, out_val=self.topk_val, group=L, stream=stream)
        return self


class PrefillPlan:
    """Preallocated buffers for one prefill chunk: many queries sharing one key range."""

    def __init__(self, dev: DeviceWorkload, k: int = 512):
        nq, max_n = dev.nq, dev.max_n
        d = dev.k_codes.device
        self.dev, self.k = dev, k
        nb = (max_n + BLOCK - 1) // BLOCK
        self.nb = nb
        self.q_codes = torch.empty(nq, 32, 64, dtype=torch.uint8, device=d)
        self.q_scales = torch.empty(nq, 32, 4, dtype=torch.uint8, device=d)
        self.block_max = torch.empty(nq, max(nb, 1), dtype=torch.float32, device=d)
        self.kb = min(k, nb)
        self.top_blocks = torch.empty(nq, k, dtype=torch.int32, device=d)
        self.block_count = torch.empty(nq, dtype=torch.int32, device=d)
        self.cand_scores = torch.empty(nq, max(self.kb * BLOCK, 1), dtype=torch.float32, device=d)
        self.topk = torch.empty(nq, k, dtype=torch.int32, device=d)
        self.topk_val = torch.empty(nq, k, dtype=torch.float32, device=d)
        self.ws_blocks = workspace(IDX_OP_BUILD_POOL, nq, max(max_n, 1), k, device=d)
        self.ws_final = workspace(IDX_OP_TOPK, nq, max(self.kb * BLOCK, 1), k, device=d)

    def run(self, stream=None, events=None):
        dv = self.dev
        idx_quantize_q(dv.q[0], dv.signs, self.q_codes, self.q_scales, stream=stream)
        if events is not None:
            events[0].record()
        idx_score_full(dv.k_codes, dv.k_scales, dv.k_base, dv.n_vis, self.q_codes, self.q_scales, dv.w[0], dv.max_n,
                       group=dv.group, block_max=self.block_max, stream=stream)
        if events is not None:
            events[1].record()
        idx_top_blocks(self.block_max, dv.n_vis, dv.max_n, self.k, self.top_blocks, self.block_count, self.ws_blocks,
                       stream=stream)
        idx_score_pool_gather(dv.k_codes, dv.k_scales, dv.k_base, dv.n_vis, self.top_blocks, self.block_count,
                              self.kb, self.q_codes, self.q_scales, dv.w[0], self.cand_scores, stream=stream)
        idx_topk(self.cand_scores, self.kb * BLOCK, self.k, self.topk, self.ws_final, out_val=self.topk_val,
                 blocks=self.top_blocks, stream=stream)
        return self


class MainKVGather:
    """Main-KV gather for core attention: the FP4 main-KV cache of `nseq` sequences of `n`
    entries each (one row per compressed position, 288 bytes) resident in HBM, and one
    idx_gather_kv per selection (a layer's top-512 of every query) into preallocated bf16
    buffers. Only the rows that the given selections touch are written at setup (quantised by
    idx_quantize_kv from the supplied bf16 rows); the rest of the cache stays zero."""

    def __init__(self, nseq: int, n: int, selections: list, rows_for, device="cuda", chunk: int = 1 << 16):
        from . import MKV_DIM, idx_quantize_kv

        self.nseq, self.n = nseq, n
        total = nseq * n
        self.codes = torch.zeros(total, MKV_DIM // 2, dtype=torch.uint8, device=device)
        self.scales = torch.zeros(total, MKV_DIM // 16, dtype=torch.uint8, device=device)
        self.kv_base = torch.arange(nseq, dtype=torch.int64, device=device) * n
        self.n_vis = torch.full((nseq,), n, dtype=torch.int32, device=device)
        self.sel = [torch.from_numpy(np.ascontiguousarray(s, dtype=np.int32)).to(device) for s in selections]
        self.out = [torch.empty(s.shape[0], s.shape[1], MKV_DIM, dtype=torch.bfloat16, device=device)
                    for s in selections]
        # the distinct cache rows the selections read, written once
        rows = np.unique(np.concatenate([(np.arange(s.shape[0])[:, None] * n + s).reshape(-1)[s.reshape(-1) >= 0]
                                         for s in selections]).astype(np.int64))
        self.rows_written = len(rows)
        for r0 in range(0, len(rows), chunk):
            part = rows[r0:r0 + chunk]
            x = torch.from_numpy(rows_for(part // n, part % n).view(np.int16)).view(torch.bfloat16).to(device)
            c, s = idx_quantize_kv(x)
            dst = torch.from_numpy(part).to(device)
            self.codes.index_copy_(0, dst, c)
            self.scales.index_copy_(0, dst, s)

    def gather(self, i: int, stream=None):
        from . import idx_gather_kv

        return idx_gather_kv(self.codes, self.scales, self.kv_base, self.n_vis, self.sel[i], out=self.out[i],
                             stream=stream)
