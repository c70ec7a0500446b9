"""The allocation-free pool entry point (idx_build_pool_noalloc) against idx_build_pool, called
through the C ABI on the GPU: two calls in a row on the library's per-GPU scratch, the second with
fewer and shorter rows, each equal to the workspace form bit for bit (block ids are index work)."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import top_fp4_lightning_amd

    return top_fp4_lightning_amd


def _pools(fx, bm: np.ndarray, nv: np.ndarray, max_n: int, keep: int):
    """(pool ids, counts) from both entry points on the same device inputs"""
    nq = bm.shape[0]
    bm_d = torch.from_numpy(bm).cuda()
    nv_d = torch.from_numpy(nv).cuda()
    stream = torch.cuda.current_stream().cuda_stream
    out = []
    for noalloc in (False, True):
        pb = torch.full((nq, keep), -7, dtype=torch.int32, device="cuda")
        pc = torch.full((nq,), -7, dtype=torch.int32, device="cuda")
        if noalloc:
            st = fx.lib.idx_build_pool_noalloc(bm_d.data_ptr(), bm_d.stride(0), nv_d.data_ptr(), nq, max_n, keep, 8,
                                               pb.data_ptr(), pb.stride(0), pc.data_ptr(), ctypes.c_void_p(stream))
        else:
            ws = fx.workspace(fx.IDX_OP_BUILD_POOL, nq, max_n, keep)
            st = fx.lib.idx_build_pool(bm_d.data_ptr(), bm_d.stride(0), nv_d.data_ptr(), nq, max_n, keep, 8,
                                       pb.data_ptr(), pb.stride(0), pc.data_ptr(), ws.data_ptr(), ws.numel(),
                                       ctypes.c_void_p(stream))
        assert st == fx.IDX_OK, fx.lib.idx_last_error().decode()
        torch.cuda.synchronize()
        out.append((pb.cpu().numpy(), pc.cpu().numpy()))
    return out


def test_noalloc_pool_equals_workspace_pool(fx):
    rng = np.random.default_rng(4242)
    # first call: 6 rows up to 2^20 positions (the long-row path, candidate lists in the scratch);
    # a row of ties, an empty row and a row of one block among them
    max_n = 1 << 20
    nq = 6
    nb = (max_n + 7) // 8
    bm = rng.standard_normal((nq, nb)).astype(np.float32)
    bm[1] = np.round(bm[1] * 2.0)
    nv = np.array([max_n, 700001, 0, 5, 300000, 131073], np.int32)
    print(f"noalloc call 1: nq={nq} max_n={max_n}", flush=True)
    (pa, ca), (pb, cb) = _pools(fx, bm, nv, max_n, 2048)
    assert np.array_equal(ca, cb) and np.array_equal(pa, pb)
    assert list(ca) == [2048, 2048, 0, 1, 2048, 2048]
    # second call: fewer, shorter rows; the scratch keeps the first call's contents
    max_n = 200000
    nq = 3
    nb = (max_n + 7) // 8
    bm = rng.standard_normal((nq, nb)).astype(np.float32)
    nv = np.array([200000, 16384 * 8 + 9, 123457], np.int32)
    print(f"noalloc call 2: nq={nq} max_n={max_n}", flush=True)
    (pa, ca), (pb, cb) = _pools(fx, bm, nv, max_n, 2048)
    assert np.array_equal(ca, cb) and np.array_equal(pa, pb)
    assert (ca == 2048).all()
