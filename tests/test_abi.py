"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and rejects
bad arguments with the documented status before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4idx.h")
LIB = os.path.join(ROOT, "top_fp4_lightning_amd", "libfp4idx.so")


@pytest.fixture(scope="module")
def fx():
    if not os.path.exists(LIB):
        import importlib.util

        spec = importlib.util.spec_from_file_location("fp4idx_build", os.path.join(ROOT, "top_fp4_lightning_amd",
                                                                                   "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build_library()
    import top_fp4_lightning_amd

    return top_fp4_lightning_amd


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["idx_quantize_q", "idx_score_full", "idx_build_pool", "idx_score_pool_gather", "idx_topk",
              "idx_last_error", "idx_abi_version", "idx_workspace_size", "idx_quantize_kv", "idx_gather_kv", "idx_mask_pool",
              "idx_topk_pool"]:
        assert n in names


def test_every_declared_symbol_is_exported(fx):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(fx.lib, n)
    assert set(fx.EXPORTS) == set(declared_functions())


def test_version_and_workspace_sizes(fx):
    assert fx.abi_version() == 1
    assert fx.workspace_size(fx.IDX_OP_TOPK, 8, 1 << 20, 512) > 0
    assert fx.workspace_size(fx.IDX_OP_TOPK, 8, 1 << 20, 512) >= 8 * (1 << 20) * 8
    assert fx.workspace_size(fx.IDX_OP_BUILD_POOL, 8, 1 << 20, 2048) < fx.workspace_size(fx.IDX_OP_TOPK, 8, 1 << 20,
                                                                                           2048)
    assert fx.workspace_size(99, 8, 100, 10) == 0
    assert fx.workspace_size(fx.IDX_OP_TOPK, 8, 100, 4096) == 0
    assert fx.workspace_size(fx.IDX_OP_TOPK, -1, 100, 10) == 0


FAKE = 0x10000  # aligned, never dereferenced: validation fails first


def call(fx, name, *args):
    st = getattr(fx.lib, name)(*args)
    return st, fx.lib.idx_last_error().decode()


def test_quantize_validation(fx):
    assert call(fx, "idx_quantize_q", None, -1, None, None, None, None)[0] == fx.IDX_EINVAL
    assert call(fx, "idx_quantize_q", None, 0, None, None, None, None)[0] == fx.IDX_OK  # empty is a no-op
    st, msg = call(fx, "idx_quantize_q", None, 5, FAKE, FAKE, FAKE, None)
    assert st == fx.IDX_EINVAL and "null" in msg
    st, msg = call(fx, "idx_quantize_q", FAKE + 2, 5, FAKE, FAKE, FAKE, None)
    assert st == fx.IDX_EALIGN


def test_score_full_validation(fx):
    f = lambda *a: call(fx, "idx_score_full", *a)[0]
    good = [FAKE, FAKE, FAKE, FAKE, 4, 1, 100, FAKE, FAKE, FAKE, FAKE, 100, FAKE, 13, None, None]
    bad = list(good); bad[10] = None; bad[12] = None  # no outputs
    assert f(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[5] = 3  # group does not divide nq
    assert f(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[11] = 99  # score stride too small
    assert f(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[13] = 12  # block-max stride too small
    assert f(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[0] = FAKE + 8  # key codes must be 16-byte aligned
    assert f(*bad) == fx.IDX_EALIGN
    bad = list(good); bad[4] = 70000
    assert f(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[2] = None
    assert f(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[6] = -5
    assert f(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[6] = (1 << 24) + 1; bad[11] = 1 << 25; bad[13] = 1 << 22
    assert f(*bad) == fx.IDX_EUNSUPPORTED


def test_build_pool_validation(fx):
    ws = fx.workspace_size(fx.IDX_OP_BUILD_POOL, 4, 100, 2048)
    f = lambda *a: call(fx, "idx_build_pool", *a)[0]
    good = [FAKE, 13, FAKE, 4, 100, 2048, 8, FAKE, 2048, FAKE, FAKE, ws, None]
    bad = list(good); bad[6] = 4
    assert f(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[5] = 4096
    assert f(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[11] = ws - 1
    assert f(*bad) == fx.IDX_EWORKSPACE
    bad = list(good); bad[10] = None
    assert f(*bad) == fx.IDX_EWORKSPACE
    bad = list(good); bad[8] = 100
    assert f(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[10] = FAKE + 4
    assert f(*bad) == fx.IDX_EALIGN


def test_build_pool_noalloc_validation(fx):
    """the allocation-free pool: same argument checks, and requests beyond its fixed scratch are
    rejected before any HIP call (so before its device address is ever resolved)"""
    f = lambda *a: call(fx, "idx_build_pool_noalloc", *a)
    good = [FAKE, 1 << 17, FAKE, 8, 1 << 20, 2048, 8, FAKE, 2048, FAKE, None]
    bad = list(good); bad[6] = 4
    assert f(*bad)[0] == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[0] = None
    assert f(*bad)[0] == fx.IDX_EINVAL
    bad = list(good); bad[8] = 100
    assert f(*bad)[0] == fx.IDX_EINVAL
    bad = list(good); bad[9] = FAKE + 2
    assert f(*bad)[0] == fx.IDX_EALIGN
    # 64 rows of 2^20 positions fit in 80 MiB; 128 rows do not
    assert fx.workspace_size(fx.IDX_OP_BUILD_POOL, 64, 1 << 20, 2048) <= 80 << 20
    assert fx.workspace_size(fx.IDX_OP_BUILD_POOL, 128, 1 << 20, 2048) > 80 << 20
    bad = list(good); bad[3] = 128
    st, msg = f(*bad)
    assert st == fx.IDX_EUNSUPPORTED and "scratch" in msg
    bad = list(good); bad[3] = 0
    assert f(*bad)[0] == fx.IDX_OK  # nothing to do


def test_top_blocks_validation(fx):
    ws = fx.workspace_size(fx.IDX_OP_BUILD_POOL, 4, 1 << 20, 512)
    f = lambda *a: call(fx, "idx_top_blocks", *a)[0]
    good = [FAKE, 1 << 17, FAKE, 4, 1 << 20, 512, 8, FAKE, 512, FAKE, FAKE, ws, None]
    bad = list(good); bad[6] = 16
    assert f(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[5] = 0
    assert f(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[8] = 511
    assert f(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[11] = ws - 1
    assert f(*bad) == fx.IDX_EWORKSPACE
    bad = list(good); bad[10] = None
    assert f(*bad) == fx.IDX_EWORKSPACE
    bad = list(good); bad[9] = FAKE + 1
    assert f(*bad) == fx.IDX_EALIGN


def test_gather_and_topk_validation(fx):
    g = lambda *a: call(fx, "idx_score_pool_gather", *a)[0]
    good = [FAKE, FAKE, FAKE, FAKE, 2, FAKE, 2048, FAKE, 2048, 8, FAKE, FAKE, FAKE, FAKE, 16384, None, None]
    bad = list(good); bad[9] = 16
    assert g(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[14] = 16383
    assert g(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[6] = 100
    assert g(*bad) == fx.IDX_EINVAL
    ws = fx.workspace_size(fx.IDX_OP_TOPK, 2, 16384, 512)
    t = lambda *a: call(fx, "idx_topk", *a)[0]
    good = [FAKE, 16384, None, 2, 16384, 512, None, 0, 8, FAKE, 512, None, FAKE, ws, None]
    bad = list(good); bad[5] = 0
    assert t(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[5] = 2049
    assert t(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[10] = 100
    assert t(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[13] = ws - 8
    assert t(*bad) == fx.IDX_EWORKSPACE
    bad = list(good); bad[6] = FAKE; bad[7] = 10  # block map stride too small
    assert t(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[6] = FAKE; bad[7] = 2048; bad[8] = 4
    assert t(*bad) == fx.IDX_EUNSUPPORTED


def test_main_kv_validation(fx):
    q = lambda *a: call(fx, "idx_quantize_kv", *a)
    assert q(None, 0, None, None, None)[0] == fx.IDX_OK  # empty is a no-op
    assert q(None, -1, None, None, None)[0] == fx.IDX_EINVAL
    assert q(FAKE, 3, None, FAKE, None)[0] == fx.IDX_EINVAL
    assert q(FAKE + 8, 3, FAKE, FAKE, None)[0] == fx.IDX_EALIGN  # bf16 rows are read 16 bytes at a time
    assert q(FAKE, 3, FAKE + 2, FAKE, None)[0] == fx.IDX_EALIGN
    g = lambda *a: call(fx, "idx_gather_kv", *a)[0]
    good = [FAKE, FAKE, FAKE, FAKE, 4, FAKE, 512, 512, FAKE, None]
    assert g(*[None, None, None, None, 0, None, 0, 0, None, None]) == fx.IDX_OK
    bad = list(good); bad[5] = None
    assert g(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[6] = 100  # idx_stride < k
    assert g(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[8] = FAKE + 8
    assert g(*bad) == fx.IDX_EALIGN
    bad = list(good); bad[2] = FAKE + 4  # kv_base is int64
    assert g(*bad) == fx.IDX_EALIGN
    bad = list(good); bad[4] = 1 << 30; bad[7] = 8
    assert g(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[4] = 70000
    assert g(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[7] = -1
    assert g(*bad) == fx.IDX_EINVAL


def test_mask_pool_validation(fx):
    m = lambda *a: call(fx, "idx_mask_pool", *a)[0]
    good = [FAKE, 4096, FAKE, 10, 4096, FAKE, 2048, FAKE, 5, 8, None]
    assert m(*[None, 0, None, 0, 0, None, 0, None, 1, 8, None]) == fx.IDX_OK  # empty is a no-op
    bad = list(good); bad[0] = None
    assert m(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[1] = 100  # score_stride < max_n
    assert m(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[8] = 3  # group does not divide nq
    assert m(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[8] = 0
    assert m(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[6] = -1
    assert m(*bad) == fx.IDX_EINVAL
    bad = list(good); bad[9] = 16
    assert m(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[3] = 70000; bad[8] = 1
    assert m(*bad) == fx.IDX_EUNSUPPORTED
    bad = list(good); bad[0] = FAKE + 2
    assert m(*bad) == fx.IDX_EALIGN


def test_topk_pool_validation(fx):
    m = lambda *a: call(fx, "idx_topk_pool", *a)[0]
    # scores, stride, n_vis, nq, max_n, pool_blocks, pool_stride, pool_count, max_blocks, group, block, k,
    # out_idx, out_stride, out_val, stream
    good = [FAKE, 4096, FAKE, 10, 4096, FAKE, 2048, FAKE, 512, 5, 8, 512, FAKE, 512, None, None]
    empty = list(good); empty[3] = 0
    assert m(*empty) == fx.IDX_OK  # no rows: a no-op
    for i, v, st in [(0, None, fx.IDX_EINVAL), (2, None, fx.IDX_EINVAL), (5, None, fx.IDX_EINVAL),
                     (7, None, fx.IDX_EINVAL), (12, None, fx.IDX_EINVAL),
                     (1, 100, fx.IDX_EINVAL),  # score_stride < max_n
                     (6, 511, fx.IDX_EINVAL),  # pool_stride < max_blocks
                     (13, 511, fx.IDX_EINVAL),  # out_stride < k
                     (9, 3, fx.IDX_EINVAL), (9, 0, fx.IDX_EINVAL),  # group must divide nq
                     (11, 0, fx.IDX_EUNSUPPORTED), (11, 2049, fx.IDX_EUNSUPPORTED),
                     (8, 2049, fx.IDX_EUNSUPPORTED), (8, -1, fx.IDX_EUNSUPPORTED),
                     (4, (1 << 28) + 1, fx.IDX_EUNSUPPORTED), (10, 16, fx.IDX_EUNSUPPORTED),
                     (0, FAKE + 2, fx.IDX_EALIGN), (14, FAKE + 2, fx.IDX_EALIGN)]:
        bad = list(good)
        bad[i] = v
        if i == 4:
            bad[1] = v
        assert m(*bad) == st, (i, v)
    bad = list(good); bad[3] = 70000; bad[9] = 1
    assert m(*bad) == fx.IDX_EUNSUPPORTED


def test_recorded_calls_replay_in_order_and_raise_on_failure(fx):
    """record() keeps the binding's library calls without running them; Recorded replays them
    in order and raises the library's status like a direct call"""
    seen = []

    def fake(status):
        def f(*args):
            seen.append((status, args))
            return status
        return f

    ok, bad = fake(fx.IDX_OK), fake(fx.IDX_EINVAL)
    with fx.record() as calls:
        fx._call(ok, 1, 2)
        fx._call(ok, 3)
    assert seen == [] and [c[1] for c in calls] == [(1, 2), (3,)]
    rep = fx.Recorded(calls)
    rep()
    rep()
    assert seen == [(0, (1, 2)), (0, (3,)), (0, (1, 2)), (0, (3,))]
    with pytest.raises(fx.IdxError):
        fx.Recorded([(ok, (5,)), (bad, (6,)), (ok, (7,))])()
    assert seen[-2:] == [(0, (5,)), (fx.IDX_EINVAL, (6,))]  # stops at the failing call
    with pytest.raises(RuntimeError):
        with fx.record():
            with fx.record():
                pass
    fx._call(ok, 9)  # recording ended with the failed nesting: calls run again
    assert seen[-1] == (0, (9,))


def test_python_binding_refuses_cpu_tensors(fx):
    import torch

    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    s = torch.ones(128, dtype=torch.int8)
    with pytest.raises(ValueError):
        fx.idx_quantize_q(x, s, torch.empty(4, 64, dtype=torch.uint8), torch.empty(4, 4, dtype=torch.uint8))


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "top_fp4_lightning_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in src and "from oracle" not in src and "liboracle" not in src, fn
                assert "orc_" not in src, fn
