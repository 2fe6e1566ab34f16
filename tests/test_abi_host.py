"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and validates descriptors / plans launches without a GPU."""
import ctypes
import os
import re

import pytest

import chunked_gated_delta_fwd_amd as gdr
from chunked_gated_delta_fwd_amd import GDR_BF16, GDR_F32, GDR_I32, describe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdr.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return gdr.library()


def header_functions():
    text = open(os.path.join(ROOT, "include", "gdr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(gdr_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert set(declared) == set(gdr.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.gdr_version() == 10300


def test_exports_match_nm():
    out = os.popen("nm -D --defined-only %s" % gdr.LIB_PATH).read()
    syms = set(re.findall(r"\b(gdr_\w+)\b", out))
    assert set(header_functions()) <= syms


# --- planning / validation with fake addresses (never dereferenced) -------------

BASE = 1 << 40


class Alloc:
    """Hands out disjoint, aligned fake device addresses."""

    def __init__(self):
        self.next = BASE

    def __call__(self, dtype, shape, strides=None, misalign=0):
        n = 1
        for s in shape:
            n *= s
        addr = self.next + misalign
        self.next += ((n * 4 + 4096) // 4096 + 1) * 4096
        return describe(addr, dtype, shape, strides)


def fwd_descs(B=1, T=256, Hk=2, Hv=4, d=128, dt=GDR_BF16, gdt=GDR_BF16, N=None, varlen=True,
              h0=True, ht=True):
    A = Alloc()
    N = N if N is not None else (3 if varlen else B)
    return dict(q=A(dt, [B, T, Hk, d]), k=A(dt, [B, T, Hk, d]), v=A(dt, [B, T, Hv, d]),
                g=A(gdt, [B, T, Hv]), beta=A(gdt, [B, T, Hv]),
                cu_seqlens=A(GDR_I32, [N + 1]) if varlen else None,
                h0=A(GDR_F32, [N, Hv, d, d]) if h0 else None, o=A(dt, [B, T, Hv, d]),
                ht=A(GDR_F32, [N, Hv, d, d]) if ht else None)


def test_plan_varlen(lib):
    p = gdr.plan(**fwd_descs(T=1000, N=5), scale=0.1)
    assert p["n_seq"] == 5 and p["hv"] == 4 and p["hk"] == 2 and p["d"] == 128
    assert p["nt_max"] == (1000 + 63) // 64 + 5
    assert p["grid_fwd"] == 5 * 4 and p["block_fwd"] == 512
    assert 0 < p["lds_fwd"] <= 160 * 1024
    assert p["workspace_bytes"] == 4 * 5 + 16 and p["varlen"] == 1


def test_plan_fixed_and_d64(lib):
    p = gdr.plan(**fwd_descs(B=4, T=512, Hk=16, Hv=16, d=64, dt=GDR_F32, gdt=GDR_F32, varlen=False))
    assert p["n_seq"] == 4 and p["workspace_bytes"] == 0 and p["varlen"] == 0 and p["d"] == 64
    assert p["lds_fwd"] < gdr.plan(**fwd_descs())["lds_fwd"]
    # f32 inputs run the token-serial fp32 kernel: 256 threads, static LDS
    assert p["block_fwd"] == 256 and p["lds_fwd"] == 4 * (2 * 16 * 64 + 3 * 64 + 1)
    p = gdr.plan(**fwd_descs(dt=GDR_F32, gdt=GDR_BF16))
    assert p["block_fwd"] == 256 and p["lds_fwd"] == 4 * (2 * 8 * 128 + 3 * 128 + 1)


def test_null_strides_equal_compact_strides(lib):
    d = fwd_descs(B=1, T=64, Hk=1, Hv=1)
    A = Alloc()
    d["q"] = A(GDR_BF16, [1, 64, 1, 128], strides=[64 * 128, 128, 128, 1])
    gdr.plan(**d)   # explicit compact strides accepted
    d["q"] = A(GDR_BF16, [1, 64, 1, 128], strides=[64 * 128, 256, 128, 1])
    with pytest.raises(gdr.GdrError) as e:
        gdr.plan(**d)
    assert e.value.status == -4 and "q" in e.value.message


@pytest.mark.parametrize("mutate,status,text", [
    (lambda d, A: d.update(q=None), -1, "q: descriptor is NULL"),
    (lambda d, A: d.update(k=A(GDR_BF16, [1, 256, 3, 128])), -2, "k: shape"),
    (lambda d, A: d.update(v=A(GDR_F32, [1, 256, 4, 128])), -3, "share one dtype"),
    (lambda d, A: d.update(g=A(GDR_I32, [1, 256, 4])), -3, "g: dtype"),
    (lambda d, A: d.update(beta=A(GDR_F32, [1, 256, 4])), -3, "beta"),
    (lambda d, A: d.update(o=A(GDR_BF16, [1, 256, 4, 64])), -2, "o: shape"),
    (lambda d, A: d.update(g=A(GDR_BF16, [1, 255, 4])), -2, "g and beta"),
    (lambda d, A: d.update(h0=A(GDR_F32, [2, 4, 128, 128])), -2, "h0: shape"),
    (lambda d, A: d.update(ht=A(GDR_BF16, [3, 4, 128, 128])), -3, "ht: dtype"),
    (lambda d, A: d.update(cu_seqlens=A(GDR_F32, [4])), -3, "cu_seqlens"),
    (lambda d, A: d.update(cu_seqlens=A(GDR_I32, [0])), -2, "at least one offset"),
    (lambda d, A: d.update(q=A(GDR_BF16, [1, 256, 2, 128], misalign=2)), -1, "aligned"),
    (lambda d, A: d.update(o=describe(d["q"].t.data + 256, GDR_BF16, [1, 256, 4, 128])), -5,
     "o overlaps"),
    (lambda d, A: d.update(ht=d["h0"]), -5, "ht overlaps"),
])
def test_rejections(lib, mutate, status, text):
    d = fwd_descs()
    mutate(d, Alloc())
    with pytest.raises(gdr.GdrError) as e:
        gdr.plan(**d)
    assert e.value.status == status, e.value
    assert text in e.value.message, e.value.message


def test_rejects_unsupported_heads(lib):
    with pytest.raises(gdr.GdrError) as e:
        gdr.plan(**fwd_descs(Hk=3, Hv=4))
    assert "multiple of Hk" in e.value.message
    with pytest.raises(gdr.GdrError) as e:
        gdr.plan(**fwd_descs(d=96))
    assert "64 or 128" in e.value.message
    d = fwd_descs(B=2, varlen=True)
    with pytest.raises(gdr.GdrError) as e:
        gdr.plan(**d)
    assert "B == 1" in e.value.message


def test_rejects_nonfinite_scale(lib):
    with pytest.raises(gdr.GdrError) as e:
        gdr.plan(**fwd_descs(), scale=float("nan"))
    assert e.value.status == -1


def test_empty_inputs_plan(lib):
    p = gdr.plan(**fwd_descs(T=0, N=2))
    assert p["total_tokens"] == 0 and p["nt_max"] == 2


def test_error_text_is_per_call(lib):
    with pytest.raises(gdr.GdrError):
        gdr.plan(**fwd_descs(d=96))
    gdr.plan(**fwd_descs())
    assert lib.gdr_last_error() == b""


def test_chunk_fwd_without_gpu_reports_device(lib):
    """On a machine without a usable gfx950 device the call fails cleanly
    before enqueuing anything."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except Exception:
        pass
    d = fwd_descs()
    rc = lib.gdr_chunk_fwd(*[None if d[n] is None else d[n].ref for n in
                             ("q", "k", "v", "g", "beta", "cu_seqlens", "h0", "o", "ht")],
                           ctypes.c_float(1.0), None)
    assert rc == -6, (rc, lib.gdr_last_error())


@pytest.mark.parametrize("n_seq,groups,order_len,status,text", [
    (65, 8, 65, -2, "1 <= N <= 64"),
    (0, 8, 0, -2, "1 <= N <= 64"),
    (10, 8, 9, -2, "order must have N"),
    (10, 0, 10, -1, "groups must be in [1, 16]"),
    (10, 17, 10, -1, "groups must be in [1, 16]"),
])
def test_dispatch_order_rejections(lib, n_seq, groups, order_len, status, text):
    A = Alloc()
    cu = A(GDR_I32, [n_seq + 1])
    order = A(GDR_I32, [order_len])
    rc = lib.gdr_dispatch_order(cu.ref, ctypes.c_int32(groups), order.ref, None)
    assert rc == status, (rc, lib.gdr_last_error())
    assert text in lib.gdr_last_error().decode()


def test_dispatch_order_rejects_alias(lib):
    A = Alloc()
    cu = A(GDR_I32, [11])
    order = describe(cu.t.data + 4, GDR_I32, [10])
    assert lib.gdr_dispatch_order(cu.ref, ctypes.c_int32(4), order.ref, None) == -5


def _ckpt_call(lib, d, hck):
    args = [d[k] for k in ("q", "k", "v", "g", "beta", "cu_seqlens", "h0", "o", "ht")]
    refs = [None if x is None else x.ref for x in args] + [None if hck is None else hck.ref]
    return lib.gdr_chunk_fwd_checkpoints(*refs, ctypes.c_float(0.1), None)


@pytest.mark.parametrize("varlen,rows_delta,dtype,status,text", [
    (True, 1, GDR_F32, -2, "h_chunks: shape"),
    (True, -1, GDR_F32, -2, "h_chunks: shape"),
    (False, 1, GDR_F32, -2, "h_chunks: shape"),
    (True, 0, GDR_BF16, -3, "h_chunks: dtype"),
])
def test_checkpoints_rejections(lib, varlen, rows_delta, dtype, status, text):
    d = fwd_descs(B=1 if varlen else 2, T=200, varlen=varlen)
    rows = (200 + 63) // 64 + 3 if varlen else 2 * ((200 + 63) // 64)
    hck = Alloc()(dtype, [rows + rows_delta, 4, 128, 128])
    assert _ckpt_call(lib, d, hck) == status
    assert text in lib.gdr_last_error().decode()


def test_checkpoints_rejects_null_and_alias(lib):
    d = fwd_descs(T=200)
    assert _ckpt_call(lib, d, None) == -1
    assert "h_chunks" in lib.gdr_last_error().decode()
    rows = (200 + 63) // 64 + 3
    hck = describe(d["o"].t.data, GDR_F32, [rows, 4, 128, 128])
    assert _ckpt_call(lib, d, hck) == -5
    assert "overlaps" in lib.gdr_last_error().decode()


def _ckpt_n_call(lib, d, hck, n):
    args = [d[k] for k in ("q", "k", "v", "g", "beta", "cu_seqlens", "h0", "o", "ht")]
    refs = [None if x is None else x.ref for x in args] + [None if hck is None else hck.ref]
    return lib.gdr_chunk_fwd_checkpoints_n(*refs, ctypes.c_int64(n), ctypes.c_float(0.1), None)


@pytest.mark.parametrize("n", [0, 8, 24, -16, 2 ** 31])
def test_checkpoints_n_rejects_bad_granularity(lib, n):
    d = fwd_descs(T=200)
    hck = Alloc()(GDR_F32, [(200 + 15) // 16 + 3, 4, 128, 128])
    assert _ckpt_n_call(lib, d, hck, n) == -1
    assert "every_n" in lib.gdr_last_error().decode()


@pytest.mark.parametrize("n,varlen", [(16, True), (48, True), (64, True), (16, False), (80, False), (1024, True)])
def test_checkpoints_n_rows(lib, n, varlen):
    """R = ceil(T/n) + N rows with cu_seqlens, B ceil(T/n) without: that
    shape passes validation (then no device: GDR_EDEVICE), one row more or
    less is GDR_ESHAPE naming the piece size."""
    B = 1 if varlen else 2
    d = fwd_descs(B=B, T=200, varlen=varlen)
    rows = (200 + n - 1) // n + 3 if varlen else B * ((200 + n - 1) // n)
    far = Alloc()
    far.next = 1 << 44   # addresses disjoint from the other tensors
    assert _ckpt_n_call(lib, d, far(GDR_F32, [rows, 4, 128, 128]), n) == -6
    for delta in (1, -1):
        assert _ckpt_n_call(lib, d, far(GDR_F32, [rows + delta, 4, 128, 128]), n) == -2
        assert "pieces of %d tokens" % n in lib.gdr_last_error().decode()
    assert _ckpt_n_call(lib, d, None, n) == -1 and "h_ckpt" in lib.gdr_last_error().decode()


def dec_descs(B=3, Hk=2, Hv=4, d=128, dt=GDR_BF16, gdt=GDR_BF16):
    A = Alloc()
    return dict(q=A(dt, [B, Hk, d]), k=A(dt, [B, Hk, d]), v=A(dt, [B, Hv, d]), g=A(gdt, [B, Hv]),
                beta=A(gdt, [B, Hv]), h=A(GDR_F32, [B, Hv, d, d]), o=A(dt, [B, Hv, d]))


def _dec_call(lib, d):
    refs = [d[key].ref for key in ("q", "k", "v", "g", "beta", "h", "o")]
    return lib.gdr_decode_step(*refs, ctypes.c_float(0.1), None)


@pytest.mark.parametrize("mutate,status,text", [
    (lambda d, A: d.update(k=A(GDR_BF16, [3, 1, 128])), -2, "k: shape"),
    (lambda d, A: d.update(v=A(GDR_F32, [3, 4, 128])), -3, "share one dtype"),
    (lambda d, A: d.update(h=A(GDR_BF16, [3, 4, 128, 128])), -3, "h: dtype"),
    (lambda d, A: d.update(h=A(GDR_F32, [3, 4, 128, 64])), -2, "h: shape"),
    (lambda d, A: d.update(g=A(GDR_BF16, [3, 5])), -2, "g and beta"),
    (lambda d, A: d.update(o=A(GDR_BF16, [3, 4, 64])), -2, "o: shape"),
    (lambda d, A: d.update(o=describe(d["h"].t.data, GDR_BF16, [3, 4, 128])), -5, "o and h overlap"),
    (lambda d, A: d.update(h=describe(d["q"].t.data, GDR_F32, [3, 4, 128, 128])), -5, "h overlaps"),
])
def test_decode_rejections(lib, mutate, status, text):
    d = dec_descs()
    mutate(d, Alloc())
    assert _dec_call(lib, d) == status
    assert text in lib.gdr_last_error().decode(), lib.gdr_last_error()


def test_decode_rejects_heads_and_dims(lib):
    assert _dec_call(lib, dec_descs(Hk=3, Hv=4)) == -2
    assert "multiple of Hk" in lib.gdr_last_error().decode()
    assert _dec_call(lib, dec_descs(d=96)) == -2
    assert "64 or 128" in lib.gdr_last_error().decode()


# --- backward and per-channel-gate entry points (validation only) ---------------

def bwd_descs(B=1, T=256, Hk=2, Hv=4, d=128, dt=GDR_BF16, N=3, dht=True, dh0=True):
    A = Alloc()   # one allocator: every descriptor is disjoint from every other
    return dict(q=A(dt, [B, T, Hk, d]), k=A(dt, [B, T, Hk, d]), v=A(dt, [B, T, Hv, d]),
                g=A(GDR_BF16, [B, T, Hv]), beta=A(GDR_BF16, [B, T, Hv]), cu_seqlens=A(GDR_I32, [N + 1]),
                h0=A(GDR_F32, [N, Hv, d, d]), do=A(dt, [B, T, Hv, d]), dht=A(GDR_F32, [N, Hv, d, d]) if dht else None,
                dq=A(dt, [B, T, Hk, d]), dk=A(dt, [B, T, Hk, d]), dv=A(dt, [B, T, Hv, d]),
                dg=A(GDR_F32, [B, T, Hv]), dbeta=A(GDR_F32, [B, T, Hv]),
                dh0=A(GDR_F32, [N, Hv, d, d]) if dh0 else None)


BWD_ORDER = ("q", "k", "v", "g", "beta", "cu_seqlens", "h0", "do", "dht", "dq", "dk", "dv", "dg", "dbeta", "dh0")


def _bwd_call(lib, d):
    return lib.gdr_chunk_bwd(*[None if d[n] is None else d[n].ref for n in BWD_ORDER], ctypes.c_float(0.1), None)


@pytest.mark.parametrize("mutate,status,text", [
    (lambda d, A: d.update(do=None), -1, "do: descriptor is NULL"),
    (lambda d, A: d.update(do=A(GDR_BF16, [1, 256, 4, 64])), -2, "do: shape"),
    (lambda d, A: d.update(do=A(GDR_F32, [1, 256, 4, 128])), -3, "share one dtype"),
    (lambda d, A: d.update(dht=A(GDR_BF16, [3, 4, 128, 128])), -3, "dht: dtype"),
    (lambda d, A: d.update(dht=A(GDR_F32, [2, 4, 128, 128])), -2, "dht: shape"),
    (lambda d, A: d.update(dq=None), -1, "dq: descriptor is NULL"),
    (lambda d, A: d.update(dq=A(GDR_F32, [1, 256, 2, 128])), -3, "dq: dtype"),
    (lambda d, A: d.update(dk=A(GDR_BF16, [1, 256, 4, 128])), -2, "dk: shape"),
    (lambda d, A: d.update(dv=A(GDR_BF16, [1, 256, 2, 128])), -2, "dv: shape"),
    (lambda d, A: d.update(dg=A(GDR_BF16, [1, 256, 4])), -3, "dg: dtype"),
    (lambda d, A: d.update(dbeta=A(GDR_F32, [1, 255, 4])), -2, "dbeta: shape"),
    (lambda d, A: d.update(dh0=A(GDR_F32, [3, 4, 64, 128])), -2, "dh0: shape"),
    (lambda d, A: d.update(dq=describe(d["q"].t.data, GDR_BF16, [1, 256, 2, 128])), -5, "overlaps an input"),
    (lambda d, A: d.update(dv=describe(d["do"].t.data, GDR_BF16, [1, 256, 4, 128])), -5, "overlaps an input"),
    (lambda d, A: d.update(dk=describe(d["dq"].t.data, GDR_BF16, [1, 256, 2, 128])), -5, "outputs overlap"),
])
def test_bwd_rejections(lib, mutate, status, text):
    d = bwd_descs()
    mutate(d, Alloc())
    assert _bwd_call(lib, d) == status, lib.gdr_last_error()
    assert text in lib.gdr_last_error().decode(), lib.gdr_last_error()


def test_bwd_accepts_optional_dht_dh0_then_needs_a_device(lib):
    """With every descriptor valid (NULL dht and dh0 allowed) the call gets as
    far as the device check."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except Exception:
        pass
    assert _bwd_call(lib, bwd_descs(dht=False, dh0=False)) == -6


KDA_ORDER = ("q", "k", "v", "g", "beta", "cu_seqlens", "h0", "o", "ht")


def _kda_call(lib, d):
    return lib.gdr_chunk_kda_fwd(*[None if d[n] is None else d[n].ref for n in KDA_ORDER], ctypes.c_float(0.1), None)


def kda_descs(B=1, T=256, Hk=2, Hv=4, d=128, dt=GDR_BF16, N=3):
    A = Alloc()
    return dict(q=A(dt, [B, T, Hk, d]), k=A(dt, [B, T, Hk, d]), v=A(dt, [B, T, Hv, d]),
                g=A(GDR_BF16, [B, T, Hv, d]), beta=A(GDR_BF16, [B, T, Hv]), cu_seqlens=A(GDR_I32, [N + 1]),
                h0=A(GDR_F32, [N, Hv, d, d]), o=A(dt, [B, T, Hv, d]), ht=A(GDR_F32, [N, Hv, d, d]))


@pytest.mark.parametrize("mutate,status,text", [
    (lambda d, A: d.update(g=A(GDR_BF16, [1, 256, 4])), -2, "g: expected 4 dimensions"),
    (lambda d, A: d.update(g=A(GDR_BF16, [1, 256, 4, 64])), -2, "g: shape"),
    (lambda d, A: d.update(g=A(GDR_F32, [1, 256, 4, 128])), -3, "g and beta must share"),
    (lambda d, A: d.update(beta=A(GDR_BF16, [1, 256, 3])), -2, "g and beta"),
    (lambda d, A: d.update(o=describe(d["g"].t.data, GDR_BF16, [1, 256, 4, 128])), -5, "o overlaps"),
    (lambda d, A: d.update(ht=describe(d["g"].t.data, GDR_F32, [3, 4, 128, 128])), -5, "ht overlaps"),
])
def test_kda_rejections(lib, mutate, status, text):
    d = kda_descs()
    mutate(d, Alloc())
    assert _kda_call(lib, d) == status, lib.gdr_last_error()
    assert text in lib.gdr_last_error().decode(), lib.gdr_last_error()


# --- debug and test options (no device needed) ----------------------------------

def test_debug_set_options(lib):
    """Known options accept their values; unknown options and out-of-range
    values are rejected with a message; nothing touches a device."""
    assert lib.gdr_debug_set(gdr.GDR_DEBUG_CHECK_CU, 1) == 0
    assert lib.gdr_debug_set(gdr.GDR_DEBUG_CHECK_CU, 0) == 0
    assert lib.gdr_debug_set(gdr.GDR_DEBUG_SPIN_LIMIT, 5) == 0
    assert lib.gdr_debug_set(gdr.GDR_DEBUG_SPIN_LIMIT, -1) == 0      # default again
    assert lib.gdr_debug_set(gdr.GDR_DEBUG_SPIN_LIMIT, 1 << 31) == -1
    assert b"2^31" in lib.gdr_last_error()
    assert lib.gdr_debug_set(gdr.GDR_DEBUG_FAIL_LAUNCHES, -3) == -1
    assert b"GDR_DEBUG_FAIL_LAUNCHES" in lib.gdr_last_error()
    assert lib.gdr_debug_set(99, 1) == -1
    assert b"unknown option 99" in lib.gdr_last_error()
    assert lib.gdr_debug_set(gdr.GDR_DEBUG_FAIL_LAUNCHES, 0) == 0
    assert lib.gdr_last_error() == b""


def test_validation_precedes_forced_launch_failure(lib):
    """With launch failures armed, a call whose descriptors are invalid still
    reports the validation error (nothing is enqueued, so nothing can fail)."""
    ds = fwd_descs()
    ds["k"] = describe(ds["k"].t.data, GDR_BF16, [1, 256, 2, 64])
    try:
        assert lib.gdr_debug_set(gdr.GDR_DEBUG_FAIL_LAUNCHES, 5) == 0
        with pytest.raises(gdr.GdrError) as e:
            gdr.plan(**ds)
        assert e.value.status == -2 and "k: shape" in e.value.message
        refs = [None if ds[n] is None else ds[n].ref
                for n in ("q", "k", "v", "g", "beta", "cu_seqlens", "h0", "o", "ht")]
        assert lib.gdr_chunk_fwd(*refs, ctypes.c_float(0.1), None) == -2
        assert b"k: shape" in lib.gdr_last_error()
    finally:
        lib.gdr_debug_set(gdr.GDR_DEBUG_FAIL_LAUNCHES, 0)


def test_device_status_argument_check(lib):
    assert lib.gdr_device_status(None, 0) == -1
    assert b"bits is NULL" in lib.gdr_last_error()


# --- independent key and value head dims -----------------------------------------

def _far():
    A = Alloc()
    A.next = 1 << 44   # addresses disjoint from the helpers' allocations
    return A


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_plan_independent_head_dims(lib, dk, dv):
    """dk and dv are each 64 or 128: v, o [.., dv], h0 and ht [N, Hv, dk, dv]."""
    A = _far()
    d = fwd_descs(d=dk)
    d.update(v=A(GDR_BF16, [1, 256, 4, dv]), o=A(GDR_BF16, [1, 256, 4, dv]),
             h0=A(GDR_F32, [3, 4, dk, dv]), ht=A(GDR_F32, [3, 4, dk, dv]))
    p = gdr.plan(**d)
    assert p["d"] == dk and p["dv"] == dv and p["block_fwd"] == 512
    d.update(ht=A(GDR_F32, [3, 4, dv, dk]))
    with pytest.raises(gdr.GdrError) as e:
        gdr.plan(**d)
    assert e.value.status == -2 and "ht: shape" in e.value.message
    # f32 inputs: the token-serial kernel's static LDS for these dims
    d = fwd_descs(d=dk, dt=GDR_F32)
    d.update(v=A(GDR_F32, [1, 256, 4, dv]), o=A(GDR_F32, [1, 256, 4, dv]),
             h0=A(GDR_F32, [3, 4, dk, dv]), ht=A(GDR_F32, [3, 4, dk, dv]))
    p = gdr.plan(**d)
    rg = 256 // (dv // 4)
    assert p["block_fwd"] == 256 and p["lds_fwd"] == 4 * (2 * rg * dv + 2 * dk + dv + 1)
    d.update(v=A(GDR_F32, [1, 256, 4, 96]), o=A(GDR_F32, [1, 256, 4, 96]))
    with pytest.raises(gdr.GdrError) as e:
        gdr.plan(**d)
    assert "dv must be 64 or 128" in e.value.message


def test_mixed_head_dims_pass_validation_of_fwd_checkpoints_and_decode(lib):
    A = _far()
    d = fwd_descs(d=128)
    d.update(v=A(GDR_BF16, [1, 256, 4, 64]), o=A(GDR_BF16, [1, 256, 4, 64]),
             h0=A(GDR_F32, [3, 4, 128, 64]), ht=A(GDR_F32, [3, 4, 128, 64]))
    args = [d[n] for n in ("q", "k", "v", "g", "beta", "cu_seqlens", "h0", "o", "ht")]
    refs = [None if x is None else x.ref for x in args]
    assert lib.gdr_chunk_fwd(*refs, ctypes.c_float(0.1), None) == -6   # valid; no device here
    hck = A(GDR_F32, [(256 + 15) // 16 + 3, 4, 128, 64])
    assert lib.gdr_chunk_fwd_checkpoints_n(*refs, hck.ref, ctypes.c_int64(16), ctypes.c_float(0.1), None) == -6
    dd = dec_descs()
    dd.update(v=A(GDR_BF16, [3, 4, 64]), o=A(GDR_BF16, [3, 4, 64]), h=A(GDR_F32, [3, 4, 128, 64]))
    assert _dec_call(lib, dd) == -6
    dd.update(h=A(GDR_F32, [3, 4, 64, 128]))
    assert _dec_call(lib, dd) == -2 and "h: shape" in lib.gdr_last_error().decode()


def test_bwd_and_kda_need_square_states(lib):
    A = _far()
    d = bwd_descs()
    d.update(v=A(GDR_BF16, [1, 256, 4, 64]), do=A(GDR_BF16, [1, 256, 4, 64]),
             h0=A(GDR_F32, [3, 4, 128, 64]))
    assert _bwd_call(lib, d) == -2
    assert "dk == dv" in lib.gdr_last_error().decode()
    k = kda_descs()
    k.update(v=A(GDR_BF16, [1, 256, 4, 64]), o=A(GDR_BF16, [1, 256, 4, 64]),
             h0=A(GDR_F32, [3, 4, 128, 64]), ht=A(GDR_F32, [3, 4, 128, 64]))
    assert _kda_call(lib, k) == -2
    assert "dk == dv" in lib.gdr_last_error().decode()
