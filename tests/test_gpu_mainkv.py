"""GPU parity of the main-KV FP4 codec (idx_quantize_kv, idx_gather_kv) against the oracle:
codes, scales and gathered bf16 values must be bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import top_fp4_lightning_amd

    return top_fp4_lightning_amd


def edge_rows() -> np.ndarray:
    rng = np.random.default_rng(21)
    rows = []
    r = rng.standard_normal(512)
    r[:16] = 0.0  # an all-zero group
    r[16:32] = -0.0
    rows.append(r)
    rows.append(rng.standard_normal(512) * 3000.0)  # scales saturate at 448, codes at 6
    rows.append(rng.standard_normal(512) * 1e-4)  # subnormal E4M3 scales
    t = np.zeros(512)  # exact midpoint ties under a non-power-of-two scale (1.125)
    for g in range(32):
        t[16 * g] = 6 * 1.125 * (1 if g % 2 else -1)
        t[16 * g + 1:16 * g + 8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * 1.125
        t[16 * g + 8:16 * g + 15] = -t[16 * g + 1:16 * g + 8]
    rows.append(t)
    rows.append(np.concatenate([rng.standard_normal(256) * 1e3, rng.standard_normal(256) * 1e-3]))
    return synth.f32_to_bf16_rne(np.stack(rows).astype(np.float32))


def test_quantize_kv_matches_oracle(fx):
    x = np.concatenate([synth.mkv_rows(31, np.arange(700) * 977), edge_rows()])
    want_c, want_s = oracle.mkv_quantize(x)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    codes, scales = fx.idx_quantize_kv(xd)
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy(), want_s)
    assert np.array_equal(codes.cpu().numpy(), want_c)


@pytest.mark.parametrize("nq,k", [(1, 1), (3, 512), (37, 100), (5, 7), (2, 1500)])
def test_gather_kv_matches_oracle(fx, nq, k):
    rng = np.random.default_rng(nq * 1000 + k)
    rows_per_seq = 2000
    codes = rng.integers(0, 256, (nq * rows_per_seq, 256), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (nq * rows_per_seq, 32), dtype=np.uint8)  # every finite E4M3 byte
    scales[::7] |= 0x80  # negative scales too
    base = np.arange(nq, dtype=np.int64) * rows_per_seq
    n = rng.integers(k, rows_per_seq + 1, nq).astype(np.int64)
    idx = synth.selections(nq + k, nq, n, k)
    idx[0, 0] = -1  # padding
    if k > 2:
        idx[0, 1] = int(n[0])  # one past the visible range
        idx[-1, -1] = -1
    want, bad = oracle.mkv_gather(codes, scales, base, n, idx)
    assert bad == 0
    out = fx.idx_gather_kv(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                           torch.from_numpy(base).cuda(), torch.from_numpy(n.astype(np.int32)).cuda(),
                           torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_quantize_then_gather_round_trip(fx):
    # the product path end to end: quantise seeded rows on the GPU, gather a selection, compare
    # with the oracle's own quantisation and gather of the same rows
    pos = np.arange(3000)
    x = synth.mkv_rows(32, pos)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    codes, scales = fx.idx_quantize_kv(xd)
    oc, os_ = oracle.mkv_quantize(x)
    idx = synth.selections(5, 2, 3000, 512)
    base = np.zeros(2, dtype=np.int64)
    n = np.full(2, 3000, dtype=np.int64)
    want, bad = oracle.mkv_gather(oc, os_, base, n, idx)
    out = fx.idx_gather_kv(codes, scales, torch.from_numpy(base).cuda(), torch.from_numpy(n.astype(np.int32)).cuda(),
                           torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    assert bad == 0 and np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), want)
