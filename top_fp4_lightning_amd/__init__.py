"""fp4idx: FP4 lightning-indexer hot path for MI355X (gfx950).

Thin ctypes binding over ``libfp4idx.so`` (C ABI in ``include/fp4idx.h``). Each function has
the name of the C entry point it calls and only marshals arguments: torch tensors supply device
memory and the current stream; every step of the indexer runs in the HIP kernels. There is no
CPU or eager fallback: importing fails if the library has not been built.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4idx.so")

IDX_OK, IDX_EINVAL, IDX_EALIGN, IDX_EUNSUPPORTED, IDX_EHIP, IDX_EWORKSPACE = 0, -1, -2, -3, -4, -5
IDX_OP_BUILD_POOL, IDX_OP_TOPK = 1, 2
HEADS, DIM, BLOCK = 32, 128, 8

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with top_fp4_lightning_amd.build.build_library() "
                      "(or __graft_entry__.build()); the indexer has no fallback path")

_P, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
lib = ctypes.CDLL(LIB_PATH)
lib.idx_abi_version.restype = _i32
lib.idx_last_error.restype = ctypes.c_char_p
lib.idx_workspace_size.argtypes = [_i32, _i32, _i64, _i32]
lib.idx_workspace_size.restype = _sz
lib.idx_quantize_q.argtypes = [_P, _i64, _P, _P, _P, _P]
lib.idx_score_full.argtypes = [_P, _P, _P, _P, _i32, _i32, _i64, _P, _P, _P, _P, _i64, _P, _i64, _P, _P]
lib.idx_build_pool.argtypes = [_P, _i64, _P, _i32, _i64, _i32, _i32, _P, _i64, _P, _P, _sz, _P]
lib.idx_build_pool_noalloc.argtypes = [_P, _i64, _P, _i32, _i64, _i32, _i32, _P, _i64, _P, _P]
lib.idx_top_blocks.argtypes = [_P, _i64, _P, _i32, _i64, _i32, _i32, _P, _i64, _P, _P, _sz, _P]
lib.idx_score_pool_gather.argtypes = [_P, _P, _P, _P, _i32, _P, _i64, _P, _i32, _i32, _P, _P, _P, _P, _i64, _P, _P]
lib.idx_topk.argtypes = [_P, _i64, _P, _i32, _i64, _i32, _P, _i64, _i32, _P, _i64, _P, _P, _sz, _P]
lib.idx_quantize_kv.argtypes = [_P, _i64, _P, _P, _P]
lib.idx_gather_kv.argtypes = [_P, _P, _P, _P, _i32, _P, _i64, _i32, _P, _P]
lib.idx_mask_pool.argtypes = [_P, _i64, _P, _i32, _i64, _P, _i64, _P, _i32, _i32, _P]
lib.idx_topk_pool.argtypes = [_P, _i64, _P, _i32, _i64, _P, _i64, _P, _i32, _i32, _i32, _i32, _P, _i64, _P, _P]
for _f in ("idx_quantize_q", "idx_score_full", "idx_build_pool", "idx_build_pool_noalloc", "idx_top_blocks",
           "idx_score_pool_gather", "idx_topk",
           "idx_quantize_kv", "idx_gather_kv", "idx_mask_pool", "idx_topk_pool"):
    getattr(lib, _f).restype = _i32

EXPORTS = ("idx_abi_version", "idx_last_error", "idx_workspace_size", "idx_quantize_q", "idx_score_full",
           "idx_build_pool", "idx_build_pool_noalloc", "idx_top_blocks", "idx_score_pool_gather", "idx_topk",
           "idx_quantize_kv",
           "idx_gather_kv", "idx_mask_pool", "idx_topk_pool")
MKV_DIM = 512


class IdxError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"fp4idx status {status}: {msg}")
        self.status = status


def _check(status: int) -> None:
    if status != IDX_OK:
        raise IdxError(status, lib.idx_last_error().decode())


_recording: list | None = None


def _call(fn, *args) -> None:
    """Run one library call and raise on a failed status, or, inside record(), only keep it."""
    if _recording is not None:
        _recording.append((fn, args))
        return
    _check(fn(*args))


class Recorded:
    """A fixed sequence of library calls with their arguments marshalled once (tensor checks,
    pointers, strides and the stream resolved when recorded): replaying costs the host one foreign
    call per launch. The tensors the calls name must keep their storage while it is in use."""

    def __init__(self, calls: list):
        self.calls = list(calls)

    def __call__(self) -> None:
        for fn, args in self.calls:
            status = fn(*args)
            if status != IDX_OK:
                raise IdxError(status, lib.idx_last_error().decode())


@contextlib.contextmanager
def record():
    """Collect the library calls made inside the block, without running them: yields a list that
    holds them afterwards (wrap it in Recorded to replay)."""
    global _recording
    if _recording is not None:
        raise RuntimeError("record() does not nest")
    calls: list = []
    _recording = calls
    try:
        yield calls
    finally:
        _recording = None


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("fp4idx tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("fp4idx tensors must be contiguous")
    return t.data_ptr()


def _rows_ptr(t: torch.Tensor | None) -> int | None:
    """A 2-D argument the library reads through its own row stride: each row contiguous."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("fp4idx tensors must live on the GPU")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("fp4idx row arguments must be 2-D with contiguous rows")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def abi_version() -> int:
    return int(lib.idx_abi_version())


def workspace_size(op: int, nq: int, max_n: int, k: int) -> int:
    return int(lib.idx_workspace_size(op, nq, max_n, k))


def workspace(op: int, nq: int, max_n: int, k: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace; the library restores its counters after every call."""
    n = workspace_size(op, nq, max_n, k)
    if n == 0:
        raise ValueError("invalid workspace request")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def idx_quantize_q(x: torch.Tensor, signs: torch.Tensor, codes: torch.Tensor | None = None,
                   scales: torch.Tensor | None = None, stream=None):
    """Rotate + MXFP4-quantise bf16 rows [..., 128] -> (codes [..., 64] u8, scales [..., 4] u8)."""
    _need(x, torch.bfloat16, "x")
    _need(signs, torch.int8, "signs")
    lead = x.shape[:-1]
    rows = x.numel() // DIM
    if codes is None:
        codes = torch.empty(*lead, 64, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(*lead, 4, dtype=torch.uint8, device=x.device)
    _call(lib.idx_quantize_q, _ptr(x), rows, _ptr(signs), _ptr(codes), _ptr(scales), _stream(stream))
    return codes, scales


def idx_score_full(k_codes, k_scales, k_base, n_vis, q_codes, q_scales, w, max_n: int, group: int = 1,
                   scores=None, block_max=None, head_dots=None, stream=None):
    """Full-layer scan. Returns (scores, block_max, head_dots) as passed (None where not requested)."""
    nq = n_vis.shape[0]
    _need(k_base, torch.int64, "k_base")
    _need(n_vis, torch.int32, "n_vis")
    _need(w, torch.float32, "w")
    ss = scores.stride(0) if scores is not None else (head_dots.shape[-1] if head_dots is not None else 0)
    bs = block_max.stride(0) if block_max is not None else 0
    _call(lib.idx_score_full, _ptr(k_codes), _ptr(k_scales), _ptr(k_base), _ptr(n_vis), nq, group, max_n,
          _ptr(q_codes), _ptr(q_scales), _ptr(w),
          _ptr(scores) if head_dots is not None else _rows_ptr(scores), ss,
          _rows_ptr(block_max), bs, _ptr(head_dots), _stream(stream))
    return scores, block_max, head_dots


def idx_build_pool(block_max, n_vis, max_n: int, pool_blocks, pool_count, ws, topk_blocks: int = 2048,
                   block: int = BLOCK, stream=None):
    nq = n_vis.shape[0]
    _need(block_max, torch.float32, "block_max")
    _need(pool_blocks, torch.int32, "pool_blocks")
    _call(lib.idx_build_pool, _rows_ptr(block_max), block_max.stride(0), _ptr(n_vis), nq, max_n, topk_blocks, block,
          _ptr(pool_blocks), pool_blocks.stride(0), _ptr(pool_count), _ptr(ws), ws.numel(),
          _stream(stream))
    return pool_blocks, pool_count


def idx_build_pool_noalloc(block_max, n_vis, max_n: int, pool_blocks, pool_count, topk_blocks: int = 2048,
                           block: int = BLOCK, stream=None):
    """idx_build_pool without a workspace (the library's fixed per-GPU scratch); allocates nothing."""
    nq = n_vis.shape[0]
    _need(block_max, torch.float32, "block_max")
    _need(pool_blocks, torch.int32, "pool_blocks")
    _call(lib.idx_build_pool_noalloc, _rows_ptr(block_max), block_max.stride(0), _ptr(n_vis), nq, max_n, topk_blocks,
          block, _ptr(pool_blocks), pool_blocks.stride(0), _ptr(pool_count),
          _stream(stream))
    return pool_blocks, pool_count


def idx_top_blocks(block_max, n_vis, max_n: int, k: int, blocks, count, ws, block: int = BLOCK, stream=None):
    """Top-k blocks by raw block maxima (no pin): ascending ids [nq, >= k] and counts [nq]."""
    nq = n_vis.shape[0]
    _need(block_max, torch.float32, "block_max")
    _need(blocks, torch.int32, "blocks")
    _call(lib.idx_top_blocks, _rows_ptr(block_max), block_max.stride(0), _ptr(n_vis), nq, max_n, k, block,
          _rows_ptr(blocks), blocks.stride(0), _ptr(count), _ptr(ws), ws.numel(), _stream(stream))
    return blocks, count


def idx_score_pool_gather(k_codes, k_scales, k_base, n_vis, blocks, block_count, max_blocks: int, q_codes,
                          q_scales, w, scores, head_dots=None, block: int = BLOCK, stream=None):
    nq = n_vis.shape[0]
    _need(scores, torch.float32, "scores")
    _call(lib.idx_score_pool_gather, _ptr(k_codes), _ptr(k_scales), _ptr(k_base), _ptr(n_vis), nq, _rows_ptr(blocks),
          blocks.stride(0), _ptr(block_count), max_blocks, block, _ptr(q_codes),
          _ptr(q_scales), _ptr(w),
          _ptr(scores) if head_dots is not None else _rows_ptr(scores), scores.stride(0),
          _ptr(head_dots),
          _stream(stream))
    return scores


def idx_topk(scores, max_n: int, k: int, out_idx, ws, n_valid=None, out_val=None, blocks=None, block: int = BLOCK,
             stream=None):
    nq = scores.shape[0]
    _need(scores, torch.float32, "scores")
    _need(out_idx, torch.int32, "out_idx")
    _call(lib.idx_topk, _rows_ptr(scores), scores.stride(0), _ptr(n_valid), nq, max_n, k, _rows_ptr(blocks),
          blocks.stride(0) if blocks is not None else 0, block, _ptr(out_idx), out_idx.stride(0),
          _ptr(out_val), _ptr(ws), ws.numel(), _stream(stream))
    return out_idx, out_val


def idx_quantize_kv(x: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                    stream=None):
    """Main-KV rows bf16 [..., 512] -> (codes [..., 256] u8, E4M3 scales [..., 32] u8)."""
    _need(x, torch.bfloat16, "x")
    lead = x.shape[:-1]
    rows = x.numel() // MKV_DIM
    if codes is None:
        codes = torch.empty(*lead, MKV_DIM // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(*lead, MKV_DIM // 16, dtype=torch.uint8, device=x.device)
    _call(lib.idx_quantize_kv, _ptr(x), rows, _ptr(codes), _ptr(scales), _stream(stream))
    return codes, scales


def idx_gather_kv(codes, scales, kv_base, n_vis, idx, out=None, k: int | None = None, stream=None):
    """Selected main-KV entries dequantised: idx int32 [nq, >= k] -> bf16 [nq, k, 512]."""
    _need(kv_base, torch.int64, "kv_base")
    _need(n_vis, torch.int32, "n_vis")
    _need(idx, torch.int32, "idx")
    nq = idx.shape[0]
    k = idx.shape[1] if k is None else k
    if out is None:
        out = torch.empty(nq, k, MKV_DIM, dtype=torch.bfloat16, device=idx.device)
    _need(out, torch.bfloat16, "out")
    _call(lib.idx_gather_kv, _ptr(codes), _ptr(scales), _ptr(kv_base), _ptr(n_vis), nq, _ptr(idx), idx.stride(0), k,
          _ptr(out), _stream(stream))
    return out


def idx_mask_pool(scores, n_vis, max_n: int, pool_blocks, pool_count, group: int = 1, block: int = BLOCK,
                  stream=None):
    """In place: -inf at every visible position outside the pooled blocks (the pool's training
    form); score row t uses pool row t // group."""
    _need(scores, torch.float32, "scores")
    _need(pool_blocks, torch.int32, "pool_blocks")
    nq = n_vis.shape[0]
    _call(lib.idx_mask_pool, _rows_ptr(scores), scores.stride(0), _ptr(n_vis), nq, max_n, _rows_ptr(pool_blocks),
          pool_blocks.stride(0), _ptr(pool_count), group, block, _stream(stream))
    return scores


def idx_topk_pool(scores, n_vis, max_n: int, pool_blocks, pool_count, max_blocks: int, k: int, out_idx,
                  out_val=None, group: int = 1, block: int = BLOCK, stream=None):
    """Top-k of full score rows over the pooled positions only (equal to idx_mask_pool then
    idx_topk, without writing the mask); score row t uses pool row t // group."""
    _need(scores, torch.float32, "scores")
    _need(pool_blocks, torch.int32, "pool_blocks")
    _need(out_idx, torch.int32, "out_idx")
    nq = n_vis.shape[0]
    _call(lib.idx_topk_pool, _rows_ptr(scores), scores.stride(0), _ptr(n_vis), nq, max_n, _rows_ptr(pool_blocks),
          pool_blocks.stride(0), _ptr(pool_count), max_blocks, group, block, k, _ptr(out_idx),
          out_idx.stride(0), _ptr(out_val), _stream(stream))
    return out_idx, out_val
