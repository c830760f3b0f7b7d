"""The C ABI: the library loads, exports every symbol include/rel_attn.h declares,
and its host-only entry points behave as documented (no GPU needed: argument
checks run before any launch)."""

import ctypes
import os
import re

import pytest

from paged_varlen_attention_gqa_amd import relattn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rel_attn.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rel_attn_[a-z_]+)\s*\(", src)))


def _header_int(name):
    m = re.search(rf"#define\s+{name}\s+\(?(-?\d+)\)?", open(HEADER).read())
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    return relattn.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) >= {"rel_attn_fwd", "rel_attn_fwd_splits", "rel_attn_fwd_lse", "rel_attn_combine",
                          "rel_attn_num_splits", "rel_attn_workspace_bytes", "rel_attn_strerror"}
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_codes_match_header():
    assert _header_int("REL_ATTN_FP32") == relattn.FP32
    assert _header_int("REL_ATTN_BF16") == relattn.BF16


@pytest.mark.parametrize("code", [0, -1, -2, -3, -4, -99])
def test_strerror(code):
    assert relattn.rel_attn_strerror(code)


def test_num_splits_range_and_errors(lib):
    for args in [(0, 64, 1, 32, 8, 8192), (0, 1, 1, 32, 4, 262144), (0, 4, 2048, 64, 8, 6144),
                 (1, 64, 512, 32, 4, 32768), (0, 2, 17, 4, 2, 70), (0, 1, 1, 8, 8, 1 << 20)]:
        r = lib.rel_attn_num_splits(*args)
        assert 1 <= r <= relattn.MAX_SPLITS, (args, r)
    assert lib.rel_attn_num_splits(1, 1, 1, 32, 4, 262144) == 1  # local: one split
    # long batch-1 decode splits many ways; short keys are never split below 256 per split
    assert lib.rel_attn_num_splits(0, 1, 1, 32, 4, 262144) >= 32
    assert lib.rel_attn_num_splits(0, 1, 1, 32, 4, 300) <= 2  # pieces of >= 256 keys
    assert lib.rel_attn_num_splits(0, 4, 2048, 64, 8, 300) == 1
    assert lib.rel_attn_num_splits(0, 0, 1, 32, 4, 100) == -1
    assert lib.rel_attn_num_splits(0, 1, 1, 30, 4, 100) == -1
    assert lib.rel_attn_num_splits(0, 1, 0, 32, 4, 100) == -1


def test_workspace_bytes(lib):
    assert lib.rel_attn_workspace_bytes(1, 100, 32, 128) == 0
    assert lib.rel_attn_workspace_bytes(4, 64, 32, 128) == 4 * 64 * 32 * 129 * 4
    assert lib.rel_attn_workspace_bytes(0, 64, 32, 128) == 0


def _fwd(lib, entry="rel_attn_fwd", **over):
    a = dict(q=1, k=1, v=1, bt=1, sl=1, cu=1, rel=1, out=1, dtype=1, T=4, B=2, maxq=2, mb=3, H=8,
             Hkv=2, D=128, NB=10, bs=16, E=4, scale=0.1, causal=1, wl=-1, wr=-1, splits=1, ws=None,
             wsb=0, need=None, stream=None, lse=1)
    a.update(over)
    ptr = lambda x: ctypes.c_void_p(x) if x else ctypes.c_void_p(0)  # noqa: E731
    need = a["need"]
    lse = [ptr(a["lse"])] if entry == "rel_attn_fwd_lse" else []
    return getattr(lib, entry)(
        ptr(a["q"]), ptr(a["k"]), ptr(a["v"]), ptr(a["bt"]), ptr(a["sl"]), ptr(a["cu"]), ptr(a["rel"]),
        ptr(a["out"]), *lse, a["dtype"], a["T"], a["B"], a["maxq"], a["mb"], a["H"], a["Hkv"], a["D"], a["NB"],
        a["bs"], a["E"], a["scale"], a["causal"], a["wl"], a["wr"], a["splits"], ptr(a["ws"]), a["wsb"],
        ctypes.byref(need) if need is not None else None, ptr(a["stream"]))


@pytest.mark.parametrize("over,code", [
    (dict(H=30, Hkv=4), -1),     # heads not divisible
    (dict(splits=0), -1),
    (dict(splits=513), -1),
    (dict(T=-1), -1),
    (dict(bs=0), -1),
    (dict(wl=-2), -1),
    (dict(causal=2), -1),
    (dict(q=0), -1),             # NULL q
    (dict(bt=0), -1),
    (dict(rel=0), -1),           # NULL bias with rel_extent > 0
    (dict(dtype=2), -2),
    (dict(D=96), -2),
    (dict(H=64, Hkv=2), -2),     # group of 32 heads
    (dict(splits=4), -3),        # no workspace
    (dict(splits=4, ws=16, wsb=100), -3),
    (dict(splits=4, ws=17, wsb=1 << 30), -1),  # misaligned workspace
])
@pytest.mark.parametrize("entry", ["rel_attn_fwd", "rel_attn_fwd_splits", "rel_attn_fwd_lse"])
def test_fwd_rejects_before_launch(lib, entry, over, code):
    assert _fwd(lib, entry, **over) == code


def test_fwd_lse_checks(lib):
    # one split runs as two: the workspace query reports two splits' worth
    need = ctypes.c_size_t(0)
    assert _fwd(lib, "rel_attn_fwd_lse", splits=1, need=need) == 0
    assert need.value == 2 * 4 * 8 * 129 * 4
    assert _fwd(lib, "rel_attn_fwd_lse", splits=1) == -3  # no workspace
    assert _fwd(lib, "rel_attn_fwd_lse", splits=4, ws=16, wsb=1 << 30, lse=0) == -1  # NULL lse
    assert _fwd(lib, "rel_attn_fwd_lse", T=0, B=0, q=0, out=0, lse=0) == 0


@pytest.mark.parametrize("entry", ["rel_attn_fwd", "rel_attn_fwd_splits", "rel_attn_fwd_lse"])
def test_fwd_workspace_query(lib, entry):
    need = ctypes.c_size_t(123)
    assert _fwd(lib, entry, splits=8, need=need) == 0
    assert need.value == 8 * 4 * 8 * 129 * 4


@pytest.mark.parametrize("entry", ["rel_attn_fwd", "rel_attn_fwd_splits", "rel_attn_fwd_lse"])
def test_fwd_empty_call_is_ok(lib, entry):
    assert _fwd(lib, entry, T=0, B=0, q=0, out=0) == 0


def _combine(lib, ws=16, wsb=1 << 30, out=16, dtype=1, T=4, H=8, D=128, splits=4):
    p = lambda x: ctypes.c_void_p(x) if x else ctypes.c_void_p(0)  # noqa: E731
    return lib.rel_attn_combine(p(ws), wsb, p(out), dtype, T, H, D, splits, None)


@pytest.mark.parametrize("over,code", [
    (dict(splits=1), -1),         # nothing to merge
    (dict(splits=513), -1),
    (dict(T=-1), -1),
    (dict(H=0), -1),
    (dict(out=0), -1),
    (dict(ws=17), -1),            # misaligned workspace
    (dict(dtype=5), -2),
    (dict(D=80), -2),
    (dict(ws=0), -3),
    (dict(wsb=4 * 4 * 8 * 129 * 4 - 1), -3),
])
def test_combine_rejects_before_launch(lib, over, code):
    assert _combine(lib, **over) == code


def test_combine_empty_call_is_ok(lib):
    assert _combine(lib, T=0, out=0) == 0


def _noalloc(lib, **over):
    a = dict(q=1, k=1, v=1, bt=1, sl=1, cu=1, rel=1, out=1, dtype=1, T=4, B=2, maxq=2, mb=3, H=8,
             Hkv=2, D=128, NB=10, bs=16, E=4, scale=0.1, causal=1, wl=-1, wr=-1, splits=4, stream=None)
    a.update(over)
    ptr = lambda x: ctypes.c_void_p(x) if x else ctypes.c_void_p(0)  # noqa: E731
    return lib.rel_attn_fwd_noalloc(
        ptr(a["q"]), ptr(a["k"]), ptr(a["v"]), ptr(a["bt"]), ptr(a["sl"]), ptr(a["cu"]), ptr(a["rel"]),
        ptr(a["out"]), a["dtype"], a["T"], a["B"], a["maxq"], a["mb"], a["H"], a["Hkv"], a["D"], a["NB"],
        a["bs"], a["E"], a["scale"], a["causal"], a["wl"], a["wr"], a["splits"], ptr(a["stream"]))


def test_noalloc_scratch_size(lib):
    assert lib.rel_attn_noalloc_scratch_bytes() == 32 << 20


@pytest.mark.parametrize("over,code", [
    (dict(H=30, Hkv=4), -1),
    (dict(splits=0), -1),
    (dict(splits=513), -1),
    (dict(q=0), -1),
    (dict(rel=0), -1),
    (dict(dtype=2), -2),
    (dict(D=96), -2),
    # a workspace of more than 32 MiB: 2 splits x 8192 tokens x 8 heads x 129 x 4 B
    (dict(splits=2, T=8192), -3),
    (dict(splits=512, T=64, H=32, Hkv=8), -3),
])
def test_noalloc_rejects_before_any_device_work(lib, over, code):
    """Every check of rel_attn_fwd_noalloc runs on the host before a device is touched."""
    assert _noalloc(lib, **over) == code


def test_noalloc_empty_call_is_ok(lib):
    assert _noalloc(lib, T=0, B=0, q=0, out=0) == 0
