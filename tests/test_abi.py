"""The C-ABI library on the CPU: it loads, exports every function include/osm.h
declares, and rejects invalid arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "osm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def abi():
    from online_softmax_08_amd import _abi
    return _abi


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(["attn_fwd", "attn_fwd_f32", "row_softmax",
                                            "osm_status_str"])


def test_library_exports_every_declared_symbol(abi):
    lib = ctypes.CDLL(abi.library_path())
    for name in _declared_functions():
        assert hasattr(lib, name), f"libosm.so does not export {name}"
    assert set(abi.EXPORTS) == set(_declared_functions())


def test_status_strings(abi):
    for st in range(0, 9):
        assert abi.osm_status_str(st) and abi.osm_status_str(st) != "unknown status"
    assert abi.osm_status_str(99) == "unknown status"


FAKE = 1 << 20  # a non-null, 16-byte aligned address; never dereferenced


def _attn_status(abi, fn, Q=FAKE, K=2 * FAKE, V=3 * FAKE, O=4 * FAKE, lse=5 * FAKE, B=1, H=1,
                 N=16, d=64, scale=0.125, causal=0):
    with pytest.raises(abi.OsmError) as e:
        getattr(abi, fn)(Q, K, V, O, lse, B, H, N, d, scale, causal)
    return e.value.status


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_f32"])
def test_attn_validation(abi, fn):
    assert _attn_status(abi, fn, d=65) == abi.OSM_ERR_HEAD_DIM
    assert _attn_status(abi, fn, d=256) == abi.OSM_ERR_HEAD_DIM
    assert _attn_status(abi, fn, B=-1) == abi.OSM_ERR_SIZE
    assert _attn_status(abi, fn, N=-5) == abi.OSM_ERR_SIZE
    assert _attn_status(abi, fn, B=1 << 16, H=1 << 16) == abi.OSM_ERR_SIZE
    assert _attn_status(abi, fn, scale=0.0) == abi.OSM_ERR_SCALE
    assert _attn_status(abi, fn, scale=-1.0) == abi.OSM_ERR_SCALE
    assert _attn_status(abi, fn, scale=float("nan")) == abi.OSM_ERR_SCALE
    assert _attn_status(abi, fn, scale=float("inf")) == abi.OSM_ERR_SCALE
    assert _attn_status(abi, fn, Q=0) == abi.OSM_ERR_NULL
    assert _attn_status(abi, fn, lse=0) == abi.OSM_ERR_NULL
    assert _attn_status(abi, fn, K=2 * FAKE + 8) == abi.OSM_ERR_ALIGN
    assert _attn_status(abi, fn, lse=5 * FAKE + 2) == abi.OSM_ERR_ALIGN
    assert _attn_status(abi, fn, O=FAKE) == abi.OSM_ERR_ALIAS           # O is Q
    assert _attn_status(abi, fn, O=3 * FAKE + 256) == abi.OSM_ERR_ALIAS  # O inside V
    assert _attn_status(abi, fn, lse=4 * FAKE + 16) == abi.OSM_ERR_ALIAS  # lse inside O


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_f32"])
def test_attn_empty_problem_is_a_noop(abi, fn):
    # Nothing to do: succeeds without touching the device, pointers may be NULL.
    getattr(abi, fn)(0, 0, 0, 0, 0, 0, 4, 128, 64, 0.125, 1)
    getattr(abi, fn)(0, 0, 0, 0, 0, 2, 4, 0, 128, 0.125, 0)


def test_softmax_validation(abi):
    def status(x, y, B, N):
        with pytest.raises(abi.OsmError) as e:
            abi.row_softmax(x, y, B, N)
        return e.value.status
    assert status(FAKE, 2 * FAKE, -1, 4) == abi.OSM_ERR_SIZE
    assert status(FAKE, 2 * FAKE, 4, -1) == abi.OSM_ERR_SIZE
    assert status(0, 2 * FAKE, 4, 8) == abi.OSM_ERR_NULL
    assert status(FAKE + 2, 2 * FAKE, 4, 8) == abi.OSM_ERR_ALIGN
    assert status(FAKE, FAKE + 4, 4, 8) == abi.OSM_ERR_ALIAS  # partial overlap
    abi.row_softmax(0, 0, 0, 8)  # empty: a valid no-op


def test_valid_call_without_a_gpu_fails_loudly(abi):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(abi.OsmError) as e:
        abi.attn_fwd(FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE, 1, 1, 16, 64, 0.125, 0)
    assert e.value.status in (abi.OSM_ERR_HIP, abi.OSM_ERR_DEVICE)
