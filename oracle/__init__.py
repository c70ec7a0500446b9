"""CPU oracle for the FP4 lightning indexer (ctypes wrapper over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the benchmark's CPU
baseline leg, never by the product package. It shares no code with the GPU library.

Every function follows the definitions stated in ``oracle.c``'s header (score equation, E2M1
value set and quantise rule, block maxima, pin, pool, mask-form Reindex from the pages).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-o", _LIB_PATH, os.path.join(_HERE, "oracle.c"),
           "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        src = os.path.join(_HERE, "oracle.c")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(src) > os.path.getmtime(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P, i64, i32, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        L.orc_inv_sqrt128_f32.restype = ctypes.c_float
        L.orc_rotate.argtypes = [P, P, P]
        L.orc_e2m1_value.argtypes = [ctypes.c_int]
        L.orc_e2m1_value.restype = d
        L.orc_e2m1_code.argtypes = [d]
        L.orc_e2m1_code.restype = ctypes.c_int
        L.orc_scale_exp.argtypes = [d]
        L.orc_scale_exp.restype = ctypes.c_int
        L.orc_quantize_row.argtypes = [P, P, P]
        L.orc_quantize_rows.argtypes = [P, i64, P, P, P, ctypes.c_int]
        L.orc_head_dot.argtypes = [P, P, P, P, P, P]
        L.orc_head_dot.restype = ctypes.c_int
        L.orc_score.argtypes = [P, P, P, P, P, P, P]
        L.orc_score.restype = d
        L.orc_score_rows.argtypes = [P, P, P, P, P, i64, P, P, P]
        L.orc_topk.argtypes = [P, i64, i32, P]
        L.orc_topk.restype = i32
        L.orc_block_max.argtypes = [P, i64, i32, P]
        L.orc_block_max.restype = i64
        L.orc_pool.argtypes = [P, i64, i32, i32, P]
        L.orc_pool.restype = i32
        L.orc_e4m3_value.argtypes = [ctypes.c_int]
        L.orc_e4m3_value.restype = d
        L.orc_e4m3_scale_for.argtypes = [d]
        L.orc_e4m3_scale_for.restype = ctypes.c_int
        L.orc_mkv_quantize_rows.argtypes = [P, i64, P, P]
        L.orc_mkv_value.argtypes = [P, P, ctypes.c_int]
        L.orc_mkv_value.restype = d
        L.orc_mkv_gather.argtypes = [P, P, P, P, P, i32, i32, i64, P]
        L.orc_mkv_gather.restype = i64
        L.orc_mask_pool.argtypes = [P, i64, P, i32, i32, P]
        L.orc_reindex_mask.argtypes = [P, i64, P, i32, i32, i32, P]
        L.orc_reindex_mask.restype = i32
        L.orc_reindex_gather.argtypes = [P, P, P, P, P, i64, P, i32, i32, i32, P]
        L.orc_reindex_gather.restype = i32
        L.orc_decode_batch.argtypes = [P, P, P, P, i32, P, P, P, i32, P, P, P, i32, i32, i32, P, P, P, P,
                                       ctypes.c_int]
        L.orc_mac_count.restype = ctypes.c_uint64
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    return max(1, os.cpu_count() or 1)


# ------------------------------------------------------------------ encoding
def inv_sqrt128_f32() -> float:
    return float(lib().orc_inv_sqrt128_f32())


def rotate(x_bf16: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """fp32 rotated rows [R, 128] of bf16 rows [R, 128]."""
    x = _c(x_bf16, np.uint16).reshape(-1, 128)
    s = _c(signs, np.int8)
    y = np.empty(x.shape, dtype=np.float32)
    for r in range(x.shape[0]):
        lib().orc_rotate(_p(x[r]), _p(s), _p(y[r]))
    return y


def e2m1_code(v: float) -> int:
    return int(lib().orc_e2m1_code(float(v)))


def e2m1_value(code: int) -> float:
    return float(lib().orc_e2m1_value(int(code)))


def scale_exp(a: float) -> int:
    return int(lib().orc_scale_exp(float(a)))


def quantize_rotated(y: np.ndarray):
    """codes [R, 64] and scales [R, 4] of already-rotated fp32 rows [R, 128]."""
    y = _c(y, np.float32).reshape(-1, 128)
    codes = np.empty((y.shape[0], 64), dtype=np.uint8)
    scales = np.empty((y.shape[0], 4), dtype=np.uint8)
    for r in range(y.shape[0]):
        lib().orc_quantize_row(_p(y[r]), _p(codes[r]), _p(scales[r]))
    return codes, scales


def quantize(x_bf16: np.ndarray, signs: np.ndarray, nthreads: int | None = None):
    """rotate + quantise bf16 rows [..., 128] -> codes [..., 64], scales [..., 4]."""
    shape = x_bf16.shape[:-1]
    x = _c(x_bf16, np.uint16).reshape(-1, 128)
    codes = np.empty((x.shape[0], 64), dtype=np.uint8)
    scales = np.empty((x.shape[0], 4), dtype=np.uint8)
    lib().orc_quantize_rows(_p(x), x.shape[0], _p(_c(signs, np.int8)), _p(codes), _p(scales),
                            nthreads or threads())
    return codes.reshape(*shape, 64), scales.reshape(*shape, 4)


# ------------------------------------------------------------------ scoring
def head_dot(qc, qs, kc, ks):
    """exact per-head dot: (value, exactly representable in fp32, exponent spread)."""
    d = np.zeros(1, dtype=np.float64)
    sp = np.zeros(1, dtype=np.int32)
    ok = lib().orc_head_dot(_p(_c(qc, np.uint8)), _p(_c(qs, np.uint8)), _p(_c(kc, np.uint8)), _p(_c(ks, np.uint8)),
                            _p(d), _p(sp))
    return float(d[0]), bool(ok), int(sp[0])


def score_rows(q_codes, q_scales, w, k_codes, k_scales, want_dots: bool = False):
    """scores I [n], tolerance scale A [n] and optionally per-head dots [32, n] of one query."""
    kc = _c(k_codes, np.uint8).reshape(-1, 64)
    ks = _c(k_scales, np.uint8).reshape(-1, 4)
    n = kc.shape[0]
    I = np.empty(n, dtype=np.float64)
    A = np.empty(n, dtype=np.float64)
    dots = np.empty((32, n), dtype=np.float64) if want_dots else None
    lib().orc_score_rows(_p(_c(q_codes, np.uint8)), _p(_c(q_scales, np.uint8)), _p(_c(w, np.float32)), _p(kc), _p(ks),
                         n, _p(I), _p(A), _p(dots) if want_dots else None)
    return (I, A, dots) if want_dots else (I, A)


# ------------------------------------------------------------------ selection
def topk(I: np.ndarray, k: int) -> np.ndarray:
    I = _c(I, np.float64)
    out = np.empty(k, dtype=np.int32)
    lib().orc_topk(_p(I), len(I), k, _p(out))
    return out


def block_max(I: np.ndarray, block: int = 8) -> np.ndarray:
    I = _c(I, np.float64)
    nb = (len(I) + block - 1) // block
    out = np.empty(max(nb, 1), dtype=np.float64)
    lib().orc_block_max(_p(I), len(I), block, _p(out))
    return out[:nb]


def pool(bm: np.ndarray, n: int, block: int = 8, topk_blocks: int = 2048) -> np.ndarray:
    """ascending block ids of the candidate pool built from raw block maxima."""
    bm = _c(bm, np.float64)
    out = np.empty(max(topk_blocks, 1), dtype=np.int32)
    cnt = lib().orc_pool(_p(bm), n, block, topk_blocks, _p(out))
    return out[:cnt].copy()


def reindex_mask(I_full: np.ndarray, pool_blocks: np.ndarray, block: int = 8, k: int = 512) -> np.ndarray:
    I_full = _c(I_full, np.float64)
    pb = _c(pool_blocks, np.int32)
    out = np.empty(k, dtype=np.int32)
    lib().orc_reindex_mask(_p(I_full), len(I_full), _p(pb), len(pb), block, k, _p(out))
    return out


def reindex_gather(q_codes, q_scales, w, k_codes, k_scales, pool_blocks, block: int = 8, k: int = 512):
    kc = _c(k_codes, np.uint8).reshape(-1, 64)
    ks = _c(k_scales, np.uint8).reshape(-1, 4)
    pb = _c(pool_blocks, np.int32)
    out = np.empty(k, dtype=np.int32)
    lib().orc_reindex_gather(_p(_c(q_codes, np.uint8)), _p(_c(q_scales, np.uint8)), _p(_c(w, np.float32)), _p(kc),
                             _p(ks), kc.shape[0], _p(pb), len(pb), block, k, _p(out))
    return out


def decode_batch(k_codes, k_scales, k_base, n_vis, q_codes, q_scales, w, rq_codes=None, rq_scales=None, rw=None,
                 k: int = 512, block: int = 8, topk_blocks: int = 2048, nthreads: int | None = None):
    """Full layer + pool + Reindex (mask form) for nq decode queries, threaded over queries."""
    kc = _c(k_codes, np.uint8)
    ks = _c(k_scales, np.uint8)
    base = _c(k_base, np.int64)
    n = _c(n_vis, np.int64)
    nq = len(n)
    layers = 0 if rq_codes is None else rq_codes.shape[0]
    out_topk = np.empty((nq, k), dtype=np.int32)
    out_pool = np.empty((nq, topk_blocks), dtype=np.int32)
    out_pool_n = np.empty(nq, dtype=np.int32)
    out_rtopk = np.empty((max(layers, 1), nq, k), dtype=np.int32)
    dummy = np.zeros(1, dtype=np.uint8)
    lib().orc_decode_batch(_p(kc), _p(ks), _p(base), _p(n), nq, _p(_c(q_codes, np.uint8)), _p(_c(q_scales, np.uint8)),
                           _p(_c(w, np.float32)), layers,
                           _p(_c(rq_codes, np.uint8)) if layers else _p(dummy),
                           _p(_c(rq_scales, np.uint8)) if layers else _p(dummy),
                           _p(_c(rw, np.float32)) if layers else _p(dummy),
                           k, block, topk_blocks, _p(out_topk), _p(out_pool), _p(out_pool_n), _p(out_rtopk),
                           nthreads or threads())
    pools = [out_pool[t, :out_pool_n[t]].copy() for t in range(nq)]
    return out_topk, pools, out_rtopk[:layers]


def mac_count() -> int:
    return int(lib().orc_mac_count())


def mac_reset() -> None:
    lib().orc_mac_reset()


# ------------------------------------------------------------------ main KV codec
MKV_DIM = 512
MKV_GROUP = 16


def e4m3_value(b: int) -> float:
    return lib().orc_e4m3_value(int(b))


def e4m3_scale_for(a: float) -> int:
    return lib().orc_e4m3_scale_for(float(a))


def mkv_quantize(x_bf16: np.ndarray):
    """bf16 bit patterns [rows, 512] -> (codes u8 [rows, 256], E4M3 scales u8 [rows, 32])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16).reshape(-1, MKV_DIM)
    rows = x.shape[0]
    codes = np.empty((rows, MKV_DIM // 2), dtype=np.uint8)
    scales = np.empty((rows, MKV_DIM // MKV_GROUP), dtype=np.uint8)
    lib().orc_mkv_quantize_rows(_p(x), rows, _p(codes), _p(scales))
    return codes, scales


def mkv_values(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp64 values [rows, 512] of stored rows."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1, MKV_DIM // 2)
    scales = np.ascontiguousarray(scales, dtype=np.uint8).reshape(-1, MKV_DIM // MKV_GROUP)
    out = np.empty((codes.shape[0], MKV_DIM))
    for r in range(codes.shape[0]):
        for c in range(MKV_DIM):
            out[r, c] = lib().orc_mkv_value(_p(codes[r]), _p(scales[r]), c)
    return out


def mkv_gather(codes, scales, base, n, idx):
    """bf16 bit patterns [nq, k, 512] of the selected rows (zeros where idx is outside [0, n)),
    and the count of values that were not exactly representable in bf16."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    base = np.ascontiguousarray(base, dtype=np.int64)
    n = np.ascontiguousarray(n, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    nq, k = idx.shape
    out = np.empty((nq, k, MKV_DIM), dtype=np.uint16)
    bad = lib().orc_mkv_gather(_p(codes), _p(scales), _p(base), _p(n), _p(idx), nq, k, k, _p(out))
    return out, int(bad)


def mask_pool(I_full: np.ndarray, pool_blocks: np.ndarray, block: int = 8) -> np.ndarray:
    """the pool applied as the official code does: -inf outside the pooled blocks (fp64)"""
    I = np.ascontiguousarray(I_full, dtype=np.float64)
    pb = np.ascontiguousarray(pool_blocks, dtype=np.int32)
    out = np.empty(len(I))
    lib().orc_mask_pool(_p(I), len(I), _p(pb), len(pb), block, _p(out))
    return out
