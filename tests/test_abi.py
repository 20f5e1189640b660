"""CPU-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status
before touching a device (no compute calls)."""
import ctypes
import os
import re

import pytest

from fp4_kv_cache_amd import csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")
OK, INVALID, UNSUP, ALIGN, WS, HIP = 0, 1, 2, 3, 4, 5
A = 0x10000          # an aligned fake device address (never dereferenced)


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(csa2_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return csa2.load()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert sorted(csa2.EXPORTS) == names


def test_version_and_accounting(L):
    assert "libcsa2" in csa2.version()
    assert csa2.entry_bytes(csa2.FMT_MAIN) == 288
    assert csa2.entry_bytes(csa2.FMT_IDX) == 68
    assert csa2.entry_bytes(csa2.FMT_SWA) == 512
    assert csa2.entry_bytes(7) == -1
    assert csa2.kv_bytes_per_token([2, 2, 2, 1]) == 890.0


def test_workspace_sizes(L):
    assert csa2.workspace_size(csa2.OP_TOPK, 4, 524288, 512) > 0
    assert csa2.workspace_size(csa2.OP_TOPK, 4, 1024, 512) == 0
    d = csa2.workspace_size(csa2.OP_DECODE, 32, 32768, 512)
    assert d >= 32 * 32768 * 4
    assert csa2.workspace_size(csa2.OP_DECODE, 8, 1 << 20, 512,
                               pool=(2048, 8)) > 0
    assert csa2.workspace_size(csa2.OP_DECODE, 1, 100, 0) == 0
    assert csa2.workspace_size(9, 1, 100, 8) == 0


def _err():
    return csa2.load().csa2_last_error().decode()


def test_pack_errors(L):
    assert L.csa2_pack_kv(9, A, 1, A, A, None) == INVALID
    assert L.csa2_pack_kv(0, A, -1, A, A, None) == INVALID
    assert L.csa2_pack_kv(0, A, 0, A, A, None) == OK          # no-op
    assert L.csa2_pack_kv(0, None, 1, A, A, None) == INVALID
    assert L.csa2_pack_kv(2, A, 1, A, A, None) == INVALID     # SWA + scales
    assert L.csa2_pack_kv(0, A, 1, A, None, None) == INVALID
    assert L.csa2_pack_kv(0, A + 4, 1, A + 4096, A + 8192, None) == ALIGN
    assert "alignment" in _err()
    assert L.csa2_pack_kv(0, A, 4, A + 16, A + 65536, None) == INVALID  # overlap


def test_topk_errors(L):
    f = L.csa2_topk
    assert f(A, 100, None, None, 1, 0, 1, None, A * 2, None, 0, None) == UNSUP
    assert f(A, 100, None, None, 1, 4096, 1, None, A * 2, None, 0, None) == UNSUP
    assert f(A, 100, None, None, 1, 8, 65, None, A * 2, None, 0, None) == UNSUP
    assert f(A, 0, None, None, 1, 8, 1, None, A * 2, None, 0, None) == INVALID
    assert f(None, 100, None, None, 1, 8, 1, None, A * 2, None, 0, None) == INVALID
    # multi-stage rows need a workspace
    assert f(A, 1 << 20, None, None, 1, 512, 1, None, A * 1024, None, 0,
             None) == WS
    assert "workspace" in _err()


def test_attention_errors(L):
    f = L.csa2_reuse_attn
    args = [A, A, 1000, A, 512, A, A, A, 1, ctypes.c_float(0.044), A * 64,
            None, 0, None]
    bad_k = list(args); bad_k[4] = 0
    assert f(*bad_k) == UNSUP
    bad_k[4] = 4096
    assert f(*bad_k) == UNSUP
    null_q = list(args); null_q[5] = None
    assert f(*null_q) == INVALID
    mis = list(args); mis[5] = A + 2
    assert f(*mis) == ALIGN
    zero_scale = list(args); zero_scale[9] = ctypes.c_float(0.0)
    assert f(*zero_scale) == INVALID
    for bad in (float("inf"), float("-inf"), float("nan")):
        inf_scale = list(args); inf_scale[9] = ctypes.c_float(bad)
        assert f(*inf_scale) == INVALID
        assert "finite" in _err()
    alias = list(args); alias[10] = A       # out == main_codes
    assert f(*alias) == INVALID
    assert f(*[a if i != 8 else 0 for i, a in enumerate(args)]) == OK  # B = 0


def test_decode_errors(L):
    f = L.csa2_sparse_attn_decode
    assert f(None, A, A, A, A, A, 1, 512, ctypes.c_float(0.04), None, A * 64,
             A * 128, A * 256, 1 << 30, None) == INVALID
    desc = csa2.CacheDesc(A, A, A, A, 0, 1000, A)
    pool = csa2.PoolOpts(2048, 8)
    # a pool without block keys
    assert f(ctypes.byref(desc), A, A, A, A, A, 1, 512, ctypes.c_float(0.04),
             ctypes.byref(pool), A * 64, A * 128, A * 256, 1 << 30,
             None) == INVALID
    bad_pool = csa2.PoolOpts(2048, 100)
    assert f(ctypes.byref(desc), A, A, A, A, A, 1, 512, ctypes.c_float(0.04),
             ctypes.byref(bad_pool), A * 64, A * 128, A * 256, 1 << 30,
             None) == UNSUP
    # workspace too small
    assert f(ctypes.byref(desc), A, A, A, A, A, 1, 512, ctypes.c_float(0.04),
             None, A * 64, A * 128, A * 256, 16, None) == WS


def test_indexer_errors(L):
    f = L.csa2_indexer_score
    assert f(5, A, A, 10, A, None, 0, A, A, 1, A * 8, None) == INVALID
    assert f(0, A, None, 10, A, None, 0, A, A, 1, A * 8, None) == INVALID
    assert f(1, A, A, 10, A, None, 0, A, A, 1, A * 8, None) == INVALID
    assert f(0, A + 8, A, 10, A, None, 0, A, A, 1, A * 8, None) == ALIGN


def test_valid_call_without_device_reports_hip_error(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    st = L.csa2_pack_kv(0, A, 1, A * 4, A * 8, None)
    assert st == HIP
    assert _err()


def test_launch_event_hook_arguments(L):
    f = L.csa2_set_launch_events
    arr = (ctypes.c_void_p * 16)()
    assert f(arr, -1) == INVALID
    assert f(arr, 17) == INVALID
    assert f(None, 2) == INVALID
    assert f(None, 0) == OK
    assert f(arr, 0) == OK
