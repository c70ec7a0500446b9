"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Input generation only: this package holds none of the method's arithmetic (no rotation,
quantisation, scoring or selection). The C core (``synth.c``) is a counter-based SplitMix64
generator with Box-Muller normals rounded to bf16, so any slice of any stream can be produced
independently (used to regenerate only the sampled rows for full-size parity checks).

Stream tags: signs 1, q 2, k 3, w 4, planted set 5, lengths 6, planting query 7,
Reindex layer l (1..4): q 10+l, w 20+l. The ``sub`` index is the query (q, w) or the
sequence (k, planted set).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

TAG_SIGNS, TAG_Q, TAG_K, TAG_W, TAG_PLANT, TAG_LEN, TAG_PLANT_Q = 1, 2, 3, 4, 5, 6, 7
TAG_MKV, TAG_SEL = 40, 41
NHEAD, DIM = 32, 128


def build(verbose: bool = False) -> str:
    """Compile libsynth.so with gcc (plain C, -O2)."""
    import subprocess

    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-o", _LIB_PATH, os.path.join(_HERE, "synth.c"), "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        src = os.path.join(_HERE, "synth.c")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(src) > os.path.getmtime(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32
        P = ctypes.c_void_p
        L.synth_normal_bf16.argtypes = [u64, u64, u64, u64, u64, P, ctypes.c_int]
        L.synth_normal_f32.argtypes = [u64, u64, u64, u64, u64, ctypes.c_double, P]
        L.synth_signs.argtypes = [u64, u64, P, ctypes.c_int]
        L.synth_lengths.argtypes = [u64, u64, i32, i64, i64, P]
        L.synth_plant_positions.argtypes = [u64, u64, u64, i64, i64, P]
        L.synth_plant_positions.restype = i64
        L.synth_apply_plant.argtypes = [P, i64, i64, P, i64, P]
        L.synth_plant_shift.argtypes = [P, P]
        L.synth_uniform.argtypes = [u64, u64, u64, u64]
        L.synth_uniform.restype = ctypes.c_double
        L.synth_bf16_rne.argtypes = [ctypes.c_double]
        L.synth_bf16_rne.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(seed: int, tag: int, sub: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    if count:
        lib().synth_normal_bf16(seed, tag, sub, start, count, _ptr(out), _threads())
    return out


def normal_f32(seed: int, tag: int, sub: int, start: int, count: int, scale: float) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    if count:
        lib().synth_normal_f32(seed, tag, sub, start, count, scale, _ptr(out))
    return out


def signs(seed: int) -> np.ndarray:
    out = np.empty(DIM, dtype=np.int8)
    lib().synth_signs(seed, TAG_SIGNS, _ptr(out), DIM)
    return out


def uniform(seed: int, tag: int, sub: int, i: int) -> float:
    return lib().synth_uniform(seed, tag, sub, i)


def bf16_rne(x: float) -> int:
    return int(lib().synth_bf16_rne(float(x)))


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """round float32 values to bf16 bit patterns, to nearest, ties to even (finite inputs)"""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


MKV_DIM = 512


def mkv_rows_of(seed: int, seqs, positions) -> np.ndarray:
    """mkv_rows for (sequence, position) pairs: sequence b's position p is row b * 2^32 + p of
    one seeded stream, so every sequence has its own rows."""
    seqs = np.asarray(seqs, dtype=np.int64).reshape(-1)
    positions = np.asarray(positions, dtype=np.int64).reshape(-1)
    return mkv_rows(seed, (seqs << 32) + positions)


def mkv_rows(seed: int, positions) -> np.ndarray:
    """Main-KV latent rows (512 values) at arbitrary positions of a seeded cache, as bf16 bit
    patterns: standard normal values scaled to unit RMS (an RMSNorm with unit weights, the
    regime the main-KV format is sized for), rounded to bf16."""
    positions = np.asarray(positions, dtype=np.int64).reshape(-1)
    out = np.empty((len(positions), MKV_DIM), dtype=np.uint16)
    for i, p in enumerate(positions):
        v = normal_f32(seed, TAG_MKV, 0, int(p) * MKV_DIM, MKV_DIM, 1.0).astype(np.float64)
        v = v / np.sqrt((v * v).mean())
        out[i] = f32_to_bf16_rne(v.astype(np.float32))
    return out


def selections(seed: int, nq: int, n, k: int) -> np.ndarray:
    """k distinct ascending positions below n[t] per row t (all of them when n[t] <= k, then -1):
    stand-ins for a top-k output when only the gather that follows it is measured."""
    n = np.broadcast_to(np.asarray(n, dtype=np.int64), (nq,))
    out = np.full((nq, k), -1, dtype=np.int32)
    for t in range(nq):
        m = int(n[t])
        if m <= k:
            out[t, :m] = np.arange(m)
            continue
        rng = np.random.default_rng([seed, TAG_SEL, t])
        out[t] = np.sort(rng.choice(m, size=k, replace=False)).astype(np.int32)
    return out


def lengths(seed: int, nseq: int, lo: int, span: int) -> np.ndarray:
    out = np.empty(nseq, dtype=np.int64)
    lib().synth_lengths(seed, TAG_LEN, nseq, lo, span, _ptr(out))
    return out


def plant_positions(seed: int, seq: int, n: int, frac: float = 0.01) -> np.ndarray:
    m = int(math.floor(frac * n + 0.5))
    out = np.empty(max(m, 1), dtype=np.int64)
    got = lib().synth_plant_positions(seed, TAG_PLANT, seq, n, m, _ptr(out))
    assert got == m
    return out[:m].copy()


def plant_shift(q_bf16_one_query: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q_bf16_one_query, dtype=np.uint16).reshape(NHEAD * DIM)
    out = np.empty(DIM, dtype=np.float64)
    lib().synth_plant_shift(_ptr(q), _ptr(out))
    return out


# --------------------------------------------------------------------------- workloads
@dataclass
class Workload:
    """A seeded indexer workload.

    Queries t = 0..nq-1 each read key rows [k_base[t], k_base[t] + n_vis[t]) of one key cache
    holding the concatenated sequences. Sequence b owns cache rows [seq_base[b], seq_base[b] +
    seq_len[b]). ``qseq[t]`` is the sequence of query t.
    """

    name: str
    seed: int
    seq_len: np.ndarray  # int64 [nseq]
    qseq: np.ndarray  # int64 [nq]
    n_vis: np.ndarray  # int64 [nq]
    layers: int = 0  # Reindex layers with their own q, w
    plant_query: np.ndarray = field(default=None)  # int64 [nseq]: query whose mean head plants keys
    k: int = 512
    block: int = 8
    topk_blocks: int = 2048
    group: int = 1  # consecutive queries that share one sequence's key range

    @property
    def nseq(self) -> int:
        return len(self.seq_len)

    @property
    def nq(self) -> int:
        return len(self.qseq)

    @property
    def seq_base(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_len)[:-1]]).astype(np.int64)

    @property
    def k_base(self) -> np.ndarray:
        return self.seq_base[self.qseq]

    @property
    def total_keys(self) -> int:
        return int(self.seq_len.sum())

    def signs(self) -> np.ndarray:
        return signs(self.seed)

    def q(self, layer: int = 0, queries=None) -> np.ndarray:
        """bf16 queries [len(queries), 32, 128]; layer 0 is the Full layer, 1..L the Reindex layers."""
        qs = range(self.nq) if queries is None else queries
        tag = TAG_Q if layer == 0 else 10 + layer
        return np.stack([normal_bf16(self.seed, tag, int(t), 0, NHEAD * DIM) for t in qs]).reshape(-1, NHEAD, DIM)

    def w(self, layer: int = 0, queries=None) -> np.ndarray:
        qs = range(self.nq) if queries is None else queries
        tag = TAG_W if layer == 0 else 20 + layer
        return np.stack([normal_f32(self.seed, tag, int(t), 0, NHEAD, 1.0 / math.sqrt(32.0)) for t in qs])

    def planted(self, b: int) -> np.ndarray:
        return plant_positions(self.seed, b, int(self.seq_len[b]))

    def keys(self, b: int, start: int = 0, count: int | None = None) -> np.ndarray:
        """bf16 key rows [count, 128] of sequence b, positions start..start+count-1, planted."""
        n = int(self.seq_len[b])
        if count is None:
            count = n - start
        assert 0 <= start and start + count <= n
        rows = normal_bf16(self.seed, TAG_K, b, start * DIM, count * DIM).reshape(count, DIM)
        pos = self.planted(b)
        if len(pos):
            shift = plant_shift(self.q(0, [int(self.plant_query[b])])[0])
            lib().synth_apply_plant(_ptr(rows), start, count, _ptr(pos), len(pos), _ptr(shift))
        return rows

    def key_rows(self, b: int, positions: np.ndarray) -> np.ndarray:
        """bf16 key rows for arbitrary positions of sequence b (random access)."""
        positions = np.asarray(positions, dtype=np.int64)
        out = np.empty((len(positions), DIM), dtype=np.uint16)
        pos = self.planted(b)
        shift = plant_shift(self.q(0, [int(self.plant_query[b])])[0]) if len(pos) else None
        for i, s in enumerate(positions):
            row = normal_bf16(self.seed, TAG_K, b, int(s) * DIM, DIM).reshape(1, DIM)
            if shift is not None:
                lib().synth_apply_plant(_ptr(row), int(s), 1, _ptr(pos), len(pos), _ptr(shift))
            out[i] = row[0]
        return out


def decode_workload(name: str, seed: int, seq_len, layers: int = 0, k: int = 512, block: int = 8,
                    topk_blocks: int = 2048) -> Workload:
    """One query per sequence that sees its whole sequence (decode)."""
    seq_len = np.asarray(seq_len, dtype=np.int64)
    nseq = len(seq_len)
    return Workload(name=name, seed=seed, seq_len=seq_len, qseq=np.arange(nseq, dtype=np.int64),
                    n_vis=seq_len.copy(), layers=layers, plant_query=np.arange(nseq, dtype=np.int64), k=k,
                    block=block, topk_blocks=topk_blocks)


def prefill_workload(name: str, seed: int, n_keys: int, n_queries: int, k: int = 512) -> Workload:
    """n_queries consecutive queries on one sequence; query i sees positions <= n_keys - n_queries + i."""
    first = n_keys - n_queries + 1
    tp = int(math.floor(uniform(seed, TAG_PLANT_Q, 0, 0) * n_queries))
    return Workload(name=name, seed=seed, seq_len=np.array([n_keys], dtype=np.int64),
                    qseq=np.zeros(n_queries, dtype=np.int64),
                    n_vis=np.arange(first, first + n_queries, dtype=np.int64), layers=0,
                    plant_query=np.array([min(tp, n_queries - 1)], dtype=np.int64), k=k, group=n_queries)


def spec_decode_workload(name: str, seed: int, seq_len, positions: int = 6, layers: int = 0,
                         k: int = 512) -> Workload:
    """Speculative verification: `positions` consecutive queries per sequence (the token plus the
    draft positions), query j of a sequence of n entries seeing positions <= n - positions + j.
    The sequence's first query plants its keys."""
    seq_len = np.asarray(seq_len, dtype=np.int64)
    nseq = len(seq_len)
    qseq = np.repeat(np.arange(nseq, dtype=np.int64), positions)
    n_vis = np.repeat(seq_len, positions) - positions + 1 + np.tile(np.arange(positions, dtype=np.int64), nseq)
    return Workload(name=name, seed=seed, seq_len=seq_len, qseq=qseq, n_vis=n_vis, layers=layers,
                    plant_query=np.arange(nseq, dtype=np.int64) * positions, k=k, group=positions)


# The five workloads the indexer is measured on (sizes from the problem statement).
def config(name: str) -> Workload:
    if name == "decode_32k":  # single decode query, N = 32768
        return decode_workload(name, 1, [32768])
    if name == "decode_batch64":  # 64 sequences, n ~ U[64K, 128K]
        return decode_workload(name, 2, lengths(2, 64, 65536, 65537))
    if name == "reindex_1m":  # 64 x 2^20, pool from the Full layer, 4 Reindex layers
        return decode_workload(name, 3, [1 << 20] * 64, layers=4)
    if name == "fullscan_1m":  # 8 x 2^20 decoder Full scan (m = 1)
        return decode_workload(name, 4, [1 << 20] * 8, layers=4)
    if name == "fullscan_512k":  # 8 x 2^19 encoder Full scan (m = 2)
        return decode_workload(name, 4, [1 << 19] * 8)
    if name == "prefill_128k":  # 4096 queries on 131072 keys, causal
        return prefill_workload(name, 5, 131072, 4096)
    if name == "spec_decode_1m":  # 8 x 2^20, the token + 5 draft positions per sequence, 4 Reindex layers
        return spec_decode_workload(name, 6, [1 << 20] * 8, positions=6, layers=4)
    if name.startswith("encoder_512k_l") and name[-1] in "012":  # encoder Full layer l: its own 8 x 2^19 keys
        return decode_workload(name, 60 + int(name[-1]), [1 << 19] * 8)
    raise KeyError(name)


def token_1m() -> tuple:
    """The indexer work of one decode token at 1M context for a batch of 8: the encoder's 3 Full
    layers (m = 2, each over its own 2^19-entry key cache) and the decoder's layer-20 Full scan
    with the candidate pool and 4 Reindex layers (m = 1, 2^20 entries)."""
    return [config(f"encoder_512k_l{i}") for i in range(3)], config("fullscan_1m")


CONFIGS = ("decode_32k", "decode_batch64", "reindex_1m", "fullscan_1m", "fullscan_512k", "prefill_128k",
           "spec_decode_1m")
