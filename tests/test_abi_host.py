"""CPU-side checks of the C ABI and the Python binding (no GPU, no kernel launches).

* libmono_decode.so loads and exports every function include/mono_decode.h declares;
  the trace build, libmono_decode_trace.so, exports those and the two of
  include/mono_trace.h, which the product library does not;
* host validation rejects bad arguments with the documented codes and a
  message, before touching the device;
* workspace-size queries;
* the binding's zero-copy page views match the oracle's geometry.
"""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mono_decode.h")
TRACE_HEADER = os.path.join(ROOT, "include", "mono_trace.h")


@pytest.fixture(scope="module")
def lib():
    import sparse_paged_decode_amd as spd

    if not os.path.exists(spd.LIB_PATH):
        from sparse_paged_decode_amd.build import build

        build()
    return spd.load_library()


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declarations_all_exported(lib):
    import sparse_paged_decode_amd as spd

    names = _declared_functions()
    assert len(names) >= 11, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert sorted(spd.EXPORTED_SYMBOLS) == names


def test_exported_symbols_are_c_names(lib):
    # extern "C": plain names, no C++ mangling
    out = os.popen(f"nm -D --defined-only {lib._name}").read()
    for n in _declared_functions():
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_trace_build_exports(lib):
    from sparse_paged_decode_amd.build import TRACE_LIB_PATH

    assert os.path.exists(TRACE_LIB_PATH), "the build makes the trace library beside the product one"
    trace = _declared_functions(TRACE_HEADER)
    assert trace == ["mono_trace_clear", "mono_trace_read"]
    tr = ctypes.CDLL(TRACE_LIB_PATH)
    for n in _declared_functions() + trace:
        assert hasattr(tr, n), f"{n} not exported by the trace library"
    product = os.popen(f"nm -D --defined-only {lib._name}").read()
    for n in trace:
        assert not re.search(rf"\b{n}$", product, flags=re.M), f"{n} must not be in the product library"


def test_version_and_error_string(lib):
    assert lib.mono_abi_version() == 1
    assert lib.mxfp4_pages_pack(None, None, None, -1, None) == -1
    assert b"n_pages" in lib.mono_last_error()
    assert lib.mxfp4_pages_pack(None, None, None, 0, None) == 0
    assert lib.mono_last_error() == b""


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first


def _topk(lib, **kw):
    a = dict(iq=FAKE, pages=FAKE, num_pages=10, bt=FAKE, bt_stride=4, sl=FAKE, B=2, T=1, k=8, sel=FAKE,
             scores=None, ws=FAKE, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.mono_index_score_topk(a["iq"], a["pages"], a["num_pages"], a["bt"], a["bt_stride"], a["sl"],
                                     a["B"], a["T"], a["k"], a["sel"], a["scores"], a["ws"], a["ws_bytes"],
                                     a["stream"])


def _pa(lib, **kw):
    a = dict(q=FAKE, kp=FAKE, vp=FAKE, num_pages=10, H=1, bt=FAKE, bt_stride=4, sl=FAKE, B=2, T=1, sel=None, k=0,
             scale=0.088, out=FAKE, ws=FAKE, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.mono_pa_decode_mxfp4(a["q"], a["kp"], a["vp"], a["num_pages"], a["H"], a["bt"], a["bt_stride"],
                                    a["sl"], a["B"], a["T"], a["sel"], a["k"], ctypes.c_float(a["scale"]), a["out"],
                                    a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize(
    "kw,code,needle",
    [
        (dict(iq=None), -1, b"NULL"),
        (dict(B=0), -1, b"B must"),
        (dict(T=0), -1, b"T must"),
        (dict(k=0), -1, b"k must"),
        (dict(k=4 * 128 + 1), -1, b"capacity"),
        (dict(bt_stride=0), -1, b"bt_stride"),
        (dict(num_pages=0), -1, b"num_pages"),
        (dict(iq=ctypes.c_void_p((1 << 20) + 2)), -1, b"alignment"),
        (dict(ws_bytes=100), -3, b"workspace"),
    ],
)
def test_topk_validation(lib, kw, code, needle):
    assert _topk(lib, **kw) == code
    assert needle in lib.mono_last_error()


@pytest.mark.parametrize(
    "kw,code,needle",
    [
        (dict(q=None), -1, b"NULL"),
        (dict(H=0), -2, b"kv_heads"),
        (dict(H=65), -2, b"kv_heads"),
        (dict(sel=FAKE, k=0), -1, b"k must"),
        (dict(scale=float("nan")), -1, b"scale"),
        (dict(scale=float("inf")), -1, b"scale"),
        (dict(out=ctypes.c_void_p((1 << 20) + 8)), -1, b"alignment"),
        (dict(ws_bytes=16), -3, b"workspace"),
    ],
)
def test_pa_validation(lib, kw, code, needle):
    assert _pa(lib, **kw) == code
    assert needle in lib.mono_last_error()


def test_workspace_sizes(lib):
    assert lib.mono_index_score_topk_workspace(0, 1, 4, 8) == 0
    assert lib.mono_index_score_topk_workspace(2, 1, 4, 8) > 0
    big = lib.mono_index_score_topk_workspace(64, 1, 256, 2048)
    # at least the fp32 scores of every token of every query token
    assert big >= 64 * 256 * 128 * 4
    assert lib.mono_pa_decode_workspace(2, 1, 1, 4, 0, 0) > 0
    assert lib.mono_pa_decode_workspace(2, 1, 0, 4, 0, 0) == 0
    assert lib.mono_pa_decode_workspace(2, 1, 1, 4, 0, 1) == 0  # sparse needs k >= 1


def test_binding_page_views_match_oracle():
    import sparse_paged_decode_amd as spd
    from oracle import mxfp4

    raw = torch.from_numpy(np.random.default_rng(0).integers(0, 256, size=5 * 2 * 8704 + 33, dtype=np.uint8))
    pool = raw.as_strided((2, 2, 8704), (2 * 8704, 8704, 1), 33)
    data, scale = spd.mxfp4_page_views(pool)
    od, os_ = mxfp4.page_views(pool.numpy())
    assert tuple(data.shape) == od.shape == (2, 2, 128, 64)
    assert tuple(scale.shape) == os_.shape == (2, 2, 128, 4)
    assert data.stride() == (2 * 8704, 8704, 64, 1) and scale.stride() == (2 * 8704, 8704, 4, 1)
    np.testing.assert_array_equal(data.numpy(), od)
    np.testing.assert_array_equal(scale.numpy(), os_)
    with pytest.raises(ValueError):
        spd.mxfp4_page_views(torch.zeros(3, 8704, dtype=torch.int8))
    with pytest.raises(ValueError):
        spd.mxfp4_page_views(torch.zeros(3, 8700, dtype=torch.uint8))
    with pytest.raises(ValueError):
        spd.mxfp4_page_views(torch.zeros(3, 2 * 8704, dtype=torch.uint8)[:, ::2])


def test_binding_rejects_bad_tables_before_launch():
    import sparse_paged_decode_amd as spd

    iq = torch.zeros(4, 128, dtype=torch.bfloat16)
    pages = torch.zeros(3, 8704, dtype=torch.uint8)
    bt = torch.zeros(2, 3, dtype=torch.int32)
    sl = torch.full((2,), 100, dtype=torch.int32)
    with pytest.raises(ValueError, match="tables not int32"):
        spd.mono_index_score_topk(iq, pages, bt.long(), sl, 8, T=2)
    with pytest.raises(ValueError, match="row-contiguous"):
        spd.mono_index_score_topk(iq, pages, torch.zeros(3, 2, dtype=torch.int32).t(), sl, 8, T=2)
    with pytest.raises(ValueError, match="tokens for"):
        spd.mono_index_score_topk(iq[:3], pages, bt, sl, 8, T=2)
    with pytest.raises(ValueError, match="shorter than the batch"):
        spd.mono_index_score_topk(iq, pages, bt[:1], sl, 8, T=2)
    with pytest.raises(ValueError, match="uint8"):
        spd.mono_index_score_topk(iq, pages.to(torch.int8), bt, sl, 8, T=2)
