"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host (before any HIP call)
with the documented status codes. Only calls that are rejected, or that are
no-ops (zero requests), are made here: nothing is launched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import linear_attention_block_amd as bha
from linear_attention_block_amd import bha_dims, bha_strides

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bha.h")

OK, NULL, DIMS, UNSUP, ALIGN, STRIDE, DTYPE, HIP = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = 0x10000000  # 16-byte aligned, never dereferenced: every call below is rejected first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bha.library_path()):
        pytest.skip("libbha.so not built")
    return bha.load_library()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(bha_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_three_path_calls():
    fns = header_functions()
    for name in ("bha_feature_map", "bha_block_forward", "bha_state_commit"):
        assert name in fns


def test_library_exports_every_header_symbol(lib):
    fns = header_functions()
    assert set(fns) == set(bha.EXPORTED_SYMBOLS)
    for name in fns:
        assert hasattr(lib, name), name


def test_library_built_from_these_sources(lib):
    # the build compiles a hash of its sources into the library; the binding
    # refuses an in-tree library built from other sources (load_library raises)
    from linear_attention_block_amd import build
    got = bha.source_hash()
    assert len(got) == 16 and all(c in "0123456789abcdef" for c in got)
    assert got == build.source_hash()


def test_version_and_status_strings(lib):
    assert bha.version() == 10000
    for st in (OK, NULL, DIMS, UNSUP, ALIGN, STRIDE, DTYPE, HIP):
        assert bha.status_string(st).startswith(("BHA_OK", "BHA_ERR"))
    assert bha.status_string(12345) == "unknown bha_status"


def test_state_record_floats(lib):
    assert bha.state_record_floats(128, 64) == 129 * 128
    assert bha.state_record_floats(64, 32) == 65 * 64
    assert bha.state_record_floats(128, 128) == 129 * 256
    assert bha.state_record_floats(96, 64) == -1
    assert bha.state_record_floats(128, 48) == -1


def _dims(**kw):
    base = dict(num_requests=4, num_heads=2, head_dim=128, feat_half=64, block_size=32,
                io_dtype=1, scale=0.0)
    base.update(kw)
    return bha_dims(**base)


def _st(req=32 * 2 * 128, tok=2 * 128, head=128):
    return bha_strides(req, tok, head)


def fwd(lib, dims, q=FAKE, k=FAKE, v=FAKE, qs=None, w=FAKE, wh=64 * 128, gamma=FAKE,
        state=FAKE, num_slots=8, slots=FAKE, out=FAKE + (1 << 24), outs=None):
    qs = qs or _st()
    outs = outs or _st()
    P = ctypes.c_void_p
    return lib.bha_block_forward(ctypes.byref(dims) if dims is not None else None, P(q), P(k), P(v),
                                 ctypes.byref(qs), P(w), wh, P(gamma), P(state), num_slots, P(slots),
                                 P(out), ctypes.byref(outs), P(0))


def commit(lib, dims, k=FAKE, v=FAKE, ks=None, w=FAKE, wh=64 * 128, state=FAKE, num_slots=8,
           slots=FAKE):
    ks = ks or _st()
    P = ctypes.c_void_p
    return lib.bha_state_commit(ctypes.byref(dims) if dims is not None else None, P(k), P(v),
                                ctypes.byref(ks), P(w), wh, P(state), num_slots, P(slots), P(0))


def fmap(lib, dims, x=FAKE, xs=None, w=FAKE, wh=64 * 128, phi=FAKE):
    xs = xs or _st()
    P = ctypes.c_void_p
    return lib.bha_feature_map(ctypes.byref(dims) if dims is not None else None, P(x),
                               ctypes.byref(xs), P(w), wh, P(phi), P(0))


@pytest.mark.parametrize("call", [fwd, commit, fmap])
def test_zero_requests_is_a_noop(lib, call):
    # nothing is read, not even the (null) pointers
    if call is fwd:
        assert fwd(lib, _dims(num_requests=0), q=0, k=0, v=0, w=0, gamma=0, state=0, slots=0, out=0) == OK
    elif call is commit:
        assert commit(lib, _dims(num_requests=0), k=0, v=0, w=0, state=0, slots=0) == OK
    else:
        assert fmap(lib, _dims(num_requests=0), x=0, w=0, phi=0) == OK


@pytest.mark.parametrize("call", [fwd, commit, fmap])
def test_null_dims(lib, call):
    assert call(lib, None) == NULL


@pytest.mark.parametrize("call", [fwd, commit, fmap])
@pytest.mark.parametrize("kw,expect", [
    (dict(io_dtype=7), DTYPE),
    (dict(num_requests=-1), DIMS),
    (dict(num_heads=0), DIMS),
    (dict(scale=-1.0), DIMS),
    (dict(scale=float("nan")), DIMS),
    (dict(scale=float("inf")), DIMS),
    (dict(head_dim=96), UNSUP),
    (dict(head_dim=256), UNSUP),
    (dict(feat_half=48), UNSUP),
    (dict(feat_half=256), UNSUP),
    (dict(block_size=0), UNSUP),
    (dict(block_size=65), UNSUP),
])
def test_bad_dims(lib, call, kw, expect):
    assert call(lib, _dims(**kw)) == expect


@pytest.mark.parametrize("name", ["q", "k", "v", "w", "gamma", "state", "slots", "out"])
def test_forward_null_pointers(lib, name):
    assert fwd(lib, _dims(), **{name: 0}) == NULL


@pytest.mark.parametrize("name", ["k", "v", "w", "state", "slots"])
def test_commit_null_pointers(lib, name):
    assert commit(lib, _dims(), **{name: 0}) == NULL


@pytest.mark.parametrize("name", ["x", "w", "phi"])
def test_feature_map_null_pointers(lib, name):
    assert fmap(lib, _dims(), **{name: 0}) == NULL


@pytest.mark.parametrize("name,off", [("q", 8), ("k", 2), ("v", 4), ("w", 8), ("state", 4),
                                      ("out", 8), ("gamma", 2), ("slots", 1)])
def test_forward_misaligned(lib, name, off):
    assert fwd(lib, _dims(), **{name: FAKE + off}) == ALIGN


def test_commit_misaligned(lib):
    assert commit(lib, _dims(), state=FAKE + 8) == ALIGN
    assert commit(lib, _dims(), k=FAKE + 2) == ALIGN


@pytest.mark.parametrize("qs", [_st(req=-256), _st(tok=2 * 128 + 4), _st(head=129)])
def test_forward_bad_input_strides(lib, qs):
    assert fwd(lib, _dims(), qs=qs) == STRIDE


def test_forward_overlapping_output_rows(lib):
    # heads 128 apart but tokens only 64 apart: rows of different tokens overlap
    assert fwd(lib, _dims(), outs=bha_strides(32 * 2 * 128, 64, 128)) == STRIDE
    # broadcast (zero) stride is fine for an input but not for the output
    assert fwd(lib, _dims(), outs=bha_strides(0, 256, 128)) == STRIDE


def test_bad_w_head_stride(lib):
    assert fwd(lib, _dims(), wh=-8) == STRIDE
    assert fwd(lib, _dims(), wh=12) == STRIDE
    assert commit(lib, _dims(), wh=4) == STRIDE


def test_bad_slot_count(lib):
    assert fwd(lib, _dims(), num_slots=0) == DIMS
    assert commit(lib, _dims(), num_slots=-3) == DIMS


def test_fp32_stride_alignment(lib):
    # float32 tokens: strides must be multiples of 4 elements
    assert fwd(lib, _dims(io_dtype=0), qs=_st(tok=2 * 128 + 2)) == STRIDE
    assert fwd(lib, _dims(io_dtype=0), qs=_st(tok=2 * 128 + 4), outs=_st(tok=2 * 128 + 4),
               out=FAKE + (1 << 26), q=FAKE, k=FAKE, v=FAKE, num_slots=0) == DIMS


def test_size_overflow(lib):
    huge = bha_strides(1 << 61, 256, 128)
    assert fwd(lib, _dims(), qs=huge) == DIMS


def prefill(lib, dims, k=FAKE, v=FAKE, ks=None, offs=FAKE, total=100, w=FAKE, wh=64 * 128, state=FAKE,
            num_slots=8, slots=FAKE):
    ks = ks or _st(req=0)
    P = ctypes.c_void_p
    return lib.bha_state_prefill(ctypes.byref(dims) if dims is not None else None, P(k), P(v),
                                 ctypes.byref(ks), P(offs), total, P(w), wh, P(state), num_slots, P(slots), P(0))


def test_prefill_validation(lib):
    assert prefill(lib, None) == NULL
    assert prefill(lib, _dims(num_requests=0), k=0, v=0, offs=0, w=0, state=0, slots=0) == OK
    assert prefill(lib, _dims(), total=0) == OK  # nothing to fold; no pointer is read
    assert prefill(lib, _dims(), total=-1) == DIMS
    assert prefill(lib, _dims(), offs=0) == NULL
    assert prefill(lib, _dims(), offs=FAKE + 2) == ALIGN
    assert prefill(lib, _dims(), k=0) == NULL
    assert prefill(lib, _dims(), v=FAKE + 8) == ALIGN
    assert prefill(lib, _dims(), ks=_st(req=0, tok=2 * 128 + 4)) == STRIDE
    assert prefill(lib, _dims(), w=0) == NULL
    assert prefill(lib, _dims(), slots=0) == NULL
    assert prefill(lib, _dims(), num_slots=0) == DIMS
    assert prefill(lib, _dims(head_dim=96)) == UNSUP
    assert prefill(lib, _dims(), total=1 << 40) == DIMS


def fwd_commit(lib, dims, q=FAKE, k=FAKE, v=FAKE, w=FAKE, gamma=FAKE, state=FAKE, num_slots=8, slots=FAKE,
               mask=0, out=FAKE + (1 << 24), qs=None, outs=None):
    qs = qs or _st()
    outs = outs or _st()
    P = ctypes.c_void_p
    return lib.bha_block_forward_commit(ctypes.byref(dims) if dims is not None else None, P(q), P(k), P(v),
                                        ctypes.byref(qs), P(w), 64 * 128, P(gamma), P(state), num_slots, P(slots),
                                        P(mask), P(out), ctypes.byref(outs), P(0))


def test_forward_commit_validation(lib):
    assert fwd_commit(lib, None) == NULL
    assert fwd_commit(lib, _dims(num_requests=0), q=0, k=0, v=0, w=0, gamma=0, state=0, slots=0, out=0) == OK
    for name in ("q", "k", "v", "w", "gamma", "state", "slots", "out"):
        assert fwd_commit(lib, _dims(), **{name: 0}) == NULL, name
    assert fwd_commit(lib, _dims(), gamma=FAKE + 2) == ALIGN
    assert fwd_commit(lib, _dims(), state=FAKE + 4) == ALIGN
    assert fwd_commit(lib, _dims(head_dim=96)) == UNSUP
    assert fwd_commit(lib, _dims(io_dtype=5)) == DTYPE
    assert fwd_commit(lib, _dims(), num_slots=0) == DIMS
    assert fwd_commit(lib, _dims(), outs=bha_strides(0, 256, 128)) == STRIDE


def prefix_attn(lib, dims, q=FAKE, k=FAKE, v=FAKE, kp=FAKE, vp=FAKE, kps=None, offs=FAKE, total=100,
                ws=0, ws_bytes=0, out=FAKE + (1 << 24), qs=None, outs=None):
    qs = qs or _st()
    outs = outs or _st()
    kps = kps or _st(req=0)
    P = ctypes.c_void_p
    return lib.bha_prefix_attention(ctypes.byref(dims) if dims is not None else None, P(q), P(k), P(v),
                                    ctypes.byref(qs), P(kp), P(vp), ctypes.byref(kps), P(offs), total, P(ws),
                                    ws_bytes, P(out), ctypes.byref(outs), P(0))


def test_prefix_attention_validation(lib):
    assert prefix_attn(lib, None) == NULL
    assert prefix_attn(lib, _dims(num_requests=0), q=0, k=0, v=0, kp=0, vp=0, offs=0, out=0) == OK
    for name in ("q", "k", "v", "kp", "vp", "offs", "out"):
        assert prefix_attn(lib, _dims(), **{name: 0}) == NULL, name
    assert prefix_attn(lib, _dims(), offs=FAKE + 2) == ALIGN
    assert prefix_attn(lib, _dims(), kp=FAKE + 8) == ALIGN
    assert prefix_attn(lib, _dims(), total=-1) == DIMS
    assert prefix_attn(lib, _dims(), total=1 << 40) == DIMS
    assert prefix_attn(lib, _dims(), kps=_st(req=0, tok=2 * 128 + 4)) == STRIDE
    assert prefix_attn(lib, _dims(), outs=bha_strides(0, 256, 128)) == STRIDE
    assert prefix_attn(lib, _dims(head_dim=96)) == UNSUP
    assert prefix_attn(lib, _dims(block_size=65)) == UNSUP
    assert prefix_attn(lib, _dims(io_dtype=3)) == DTYPE
    assert prefix_attn(lib, _dims(), ws=FAKE + 8, ws_bytes=1 << 20) == ALIGN
    assert prefix_attn(lib, _dims(), ws=FAKE, ws_bytes=-1) == DIMS


def test_prefix_attention_workspace_size(lib):
    ws = lib.bha_prefix_attention_workspace
    # few pairs with long prefixes: split; many pairs: no split
    part = (32 * 128 + 64) * 4
    n = ws(ctypes.byref(_dims(num_requests=1, num_heads=16)), 32768)
    assert n > 0 and n % (16 * part) == 0 and n // (16 * part) <= 64
    assert ws(ctypes.byref(_dims(num_requests=256, num_heads=16)), 256 * 4096) == 0
    # short prefixes are not split (fewer than 16 chunks of 32 keys per split)
    assert ws(ctypes.byref(_dims(num_requests=1, num_heads=16)), 100) == 0
    # the float32 path splits the same way into the same fp32 partial records
    assert ws(ctypes.byref(_dims(num_requests=1, num_heads=16, io_dtype=0)), 32768) == n
    assert ws(ctypes.byref(_dims(num_requests=0)), 10) == 0
    assert ws(ctypes.byref(_dims(head_dim=96)), 10) == UNSUP
    assert ws(ctypes.byref(_dims()), -1) == DIMS
    assert ws(None, 10) == NULL


def fwd_gqa(lib, dims, hk=1, q=FAKE, k=FAKE, v=FAKE, w=FAKE, gamma=FAKE, state=FAKE, num_slots=8, slots=FAKE,
            out=FAKE + (1 << 24), qs=None, kvs=None, outs=None):
    qs = qs or _st()
    kvs = kvs or _st(req=32 * hk * 128, tok=hk * 128)
    outs = outs or _st()
    P = ctypes.c_void_p
    return lib.bha_block_forward_gqa(ctypes.byref(dims) if dims is not None else None, hk, P(q), ctypes.byref(qs),
                                     P(k), P(v), ctypes.byref(kvs), P(w), 64 * 128, P(gamma), P(state), num_slots,
                                     P(slots), P(out), ctypes.byref(outs), P(0))


def test_forward_gqa_validation(lib):
    # _dims() has 2 query heads
    assert fwd_gqa(lib, None) == NULL
    assert fwd_gqa(lib, _dims(num_requests=0), q=0, k=0, v=0, w=0, gamma=0, state=0, slots=0, out=0) == OK
    for hk in (0, -1, 3, 4):
        assert fwd_gqa(lib, _dims(), hk=hk) == DIMS, hk
    for name in ("q", "k", "v", "w", "gamma", "state", "slots", "out"):
        assert fwd_gqa(lib, _dims(), **{name: 0}) == NULL, name
    assert fwd_gqa(lib, _dims(), gamma=FAKE + 2) == ALIGN
    assert fwd_gqa(lib, _dims(), k=FAKE + 4) == ALIGN
    assert fwd_gqa(lib, _dims(), kvs=_st(tok=128 + 4)) == STRIDE
    assert fwd_gqa(lib, _dims(), num_slots=0) == DIMS
    assert fwd_gqa(lib, _dims(head_dim=96)) == UNSUP
    assert fwd_gqa(lib, _dims(), outs=bha_strides(0, 256, 128)) == STRIDE


# ------------------------------------------------------------------ streaming probe library
PROBE_HEADER = os.path.join(ROOT, "include", "bha_probe.h")


def test_probe_library_exports_every_header_symbol():
    from linear_attention_block_amd import probe

    if not os.path.exists(probe.LIB_PATH):
        pytest.skip("libbha_probe.so not built")
    src = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    fns = sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(bha_probe_\w+)\s*\(", src, flags=re.M)))
    assert fns == ["bha_probe_sink_floats", "bha_probe_stream", "bha_probe_trip_read_bytes",
                   "bha_probe_trip_write_bytes"]
    plib = probe.load_library()
    for name in fns:
        assert hasattr(plib, name), name


def test_probe_rejects_bad_arguments_on_the_host():
    from linear_attention_block_amd import probe

    if not os.path.exists(probe.LIB_PATH):
        pytest.skip("libbha_probe.so not built")
    plib = probe.load_library()
    good = probe.cfg(16, 1, 1, 2, 2)
    assert plib.bha_probe_trip_read_bytes(ctypes.byref(good)) == 4 * 16 * 1024
    assert plib.bha_probe_trip_write_bytes(ctypes.byref(good)) == 4 * 2 * 1024
    P = ctypes.c_void_p
    for bad in (probe.cfg(12, 1, 1, 2, 0), probe.cfg(16, 3, 1, 2, 0), probe.cfg(16, 1, 2, 2, 0),
                probe.cfg(16, 1, 1, 0, 0), probe.cfg(16, 1, 1, 9, 0), probe.cfg(16, 1, 1, 2, 9),
                probe.cfg(16, 1, 1, 2, 1, 5), probe.cfg(16, 1, 1, 2, 1, -1)):
        assert plib.bha_probe_trip_read_bytes(ctypes.byref(bad)) == -1
        assert plib.bha_probe_stream(ctypes.byref(bad), P(FAKE), 1, P(FAKE), P(FAKE), None) == -1
    assert plib.bha_probe_stream(None, P(FAKE), 1, P(FAKE), P(FAKE), None) == -1
    assert plib.bha_probe_stream(ctypes.byref(good), None, 1, P(FAKE), P(FAKE), None) == -1
    assert plib.bha_probe_stream(ctypes.byref(good), P(FAKE), 0, P(FAKE), P(FAKE), None) == -1
    assert plib.bha_probe_stream(ctypes.byref(good), P(FAKE), 1, None, P(FAKE), None) == -1  # stores need dst
    assert plib.bha_probe_stream(ctypes.byref(good), P(FAKE + 8), 1, P(FAKE), P(FAKE), None) == -1
