"""Host-side tests of the C ABI (no GPU needed).

They load libqlora.so, check that it exports every function include/*.h
declares, exercise the host-only entry points, and drive every argument-error
path, all of which return before the library's first HIP call.
"""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

from bit_quantized_lora_02_amd import binding as B
from conftest import gpu_available

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from bit_quantized_lora_02_amd import build as _build
        _build.build()
    return B.load_library()


def _declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared, "no declarations found"
    assert sorted(B.EXPORTED) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_storage_sizes(lib, oracle):
    for n_out, n_in in [(256, 256), (4096, 4096), (5, 4160), (28672, 8192), (1, 64)]:
        assert B.storage_bytes(n_out, n_in) == oracle.storage_bytes(n_out, n_in)
    cb, qb, sb = B.storage_bytes(4096, 4096)
    assert 8.0 * (cb + qb + sb) / 4096 ** 2 == 4.126953125


def test_codebook_matches_oracle_bitwise(lib, oracle):
    got = np.array(B.codebook(), np.float32)
    assert np.array_equal(got.view(np.uint32), oracle.nf4_levels().view(np.uint32))


def test_workspace_never_scales_with_weight(lib):
    T, r = 2048, 16
    small = B.workspace_bytes(B.OP_FWD, T, 4096, 4096, r)
    big = B.workspace_bytes(B.OP_FWD, T, 4096, 16 * 4096, r)
    # forward workspace is O(T*r + n_out*r): 16x more input features adds no weight-sized buffer
    assert big <= small * 4
    deq_bytes = 2 * 4096 * 16 * 4096  # what a stored bf16 W' would take
    assert big < deq_bytes // 100


def test_few_token_workspace_holds_the_partials_and_fits_the_static_array(lib):
    """The few-token forward writes one binary32 partial of Y per part of the reduction: 2048 columns up to
    32 tokens, 1024 from 33 to 64 with the 32-token kernel (n_in 8192: 4 and 8 parts), 4096 for one token
    (2 parts); its workspace must hold them, and every configured forward must fit the allocation-free
    entry point's 128 MiB array."""
    for T, parts in ((1, 2), (8, 4), (32, 4), (33, 8), (64, 8)):
        for n_out in (8192, 28672):
            ws = B.workspace_bytes(B.OP_FWD, T, n_out, 8192, 16)
            assert ws >= parts * T * n_out * 4, (T, n_out)
            assert ws < (parts + 2) * T * n_out * 4 + (8 << 20), (T, n_out)  # partials dominate
    shapes = [(n, k, t, r) for n, k in ((8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672))
              for t, r in ((4096, 64),)] + [(4096, 4096, 2048, 16), (14336, 4096, 4096, 64), (4096, 14336, 4096, 64)]
    shapes += [(n, 8192, t, 16) for n in (8192, 28672) for t in (1, 8, 32, 64, 128)]
    assert max(B.workspace_bytes(B.OP_FWD, t, n, k, r) for n, k, t, r in shapes) <= 128 << 20


def _nf4(n_out, n_in, p=0x1000):
    return B._NF4(n_out, n_in, p, p, p)


def _err(fn, *args):
    rc = fn(*args)
    return rc, B.load_library().qlora_last_error().decode()


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every check below fails first
MIS = ctypes.c_void_p(0x10008)


def test_error_paths_storage_and_workspace(lib):
    c = ctypes.c_size_t()
    assert lib.qlora_nf4_storage(4, 100, ctypes.byref(c), ctypes.byref(c), ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_nf4_storage(0, 64, ctypes.byref(c), ctypes.byref(c), ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_nf4_storage(4, 64, None, ctypes.byref(c), ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_workspace_bytes(7, 1, 64, 64, 8, ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_workspace_bytes(0, 1, 64, 64, 0, ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_workspace_bytes(0, 1, 64, 64, 129, ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_workspace_bytes(0, 1, 60, 64, 8, ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_workspace_bytes(0, -1, 64, 64, 8, ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_nf4_codebook(None) == B.QLORA_EINVAL
    assert B.codebook()  # still fine afterwards


def test_size_limits_keep_launches_below_2_32_work_items(lib):
    """At most 2^34 weights (the dequantization runs n / 8 work-items) and T x n_out, T x n_in below 2^32
    (the ordered finalize of a split reduction runs one work-item per output element)."""
    c = ctypes.c_size_t()
    big = 1 << 22
    assert lib.qlora_nf4_storage(1 << 12, 1 << 22, ctypes.byref(c), ctypes.byref(c), ctypes.byref(c)) == B.QLORA_OK
    assert lib.qlora_nf4_storage(big, big, ctypes.byref(c), ctypes.byref(c), ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_nf4_storage((1 << 12) + 8, 1 << 22, ctypes.byref(c), ctypes.byref(c),
                                 ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_workspace_bytes(B.OP_FWD, 1 << 10, 1 << 21, 64, 8, ctypes.byref(c)) == B.QLORA_OK
    assert lib.qlora_workspace_bytes(B.OP_FWD, 1 << 11, 1 << 21, 64, 8, ctypes.byref(c)) == B.QLORA_EINVAL
    assert lib.qlora_workspace_bytes(B.OP_BWD, 1 << 11, 64, 1 << 21, 8, ctypes.byref(c)) == B.QLORA_EINVAL
    q = _nf4(1 << 21, 64)
    FAKE = ctypes.c_void_p(0x1000)
    rc, msg = _err(lib.qlora_linear_fwd, FAKE, 1 << 11, ctypes.byref(q), FAKE, FAKE, 8, 16.0, FAKE, None, FAKE,
                   1 << 40, None)
    assert rc == B.QLORA_EINVAL and "2^32" in msg


def test_error_paths_quantize_dequant(lib):
    q = _nf4(64, 64)
    rc, msg = _err(lib.qlora_quantize_nf4, None, ctypes.byref(q), None)
    assert rc == B.QLORA_EINVAL and "W" in msg
    rc, _ = _err(lib.qlora_quantize_nf4, MIS, ctypes.byref(q), None)
    assert rc == B.QLORA_EINVAL
    bad = _nf4(64, 96)
    rc, msg = _err(lib.qlora_quantize_nf4, FAKE, ctypes.byref(bad), None)
    assert rc == B.QLORA_EINVAL and "64" in msg
    nul = B._NF4(64, 64, 0x1000, None, 0x1000)
    assert lib.qlora_quantize_nf4(FAKE, ctypes.byref(nul), None) == B.QLORA_EINVAL
    mis = B._NF4(64, 64, 0x1004, 0x1000, 0x1000)
    assert lib.qlora_quantize_nf4(FAKE, ctypes.byref(mis), None) == B.QLORA_EINVAL
    assert lib.qlora_quantize_nf4(FAKE, None, None) == B.QLORA_EINVAL
    assert lib.qlora_dequant(ctypes.byref(q), None, None) == B.QLORA_EINVAL
    assert lib.qlora_dequant(ctypes.byref(q), MIS, None) == B.QLORA_EINVAL


def _fwd(lib, X=FAKE, T=4, q=None, A=FAKE, Bm=FAKE, r=8, alpha=16.0, Y=FAKE, U=None, ws=FAKE, nb=1 << 30):
    q = q if q is not None else _nf4(64, 64)
    return lib.qlora_linear_fwd(X, T, ctypes.byref(q), A, Bm, r, alpha, Y, U, ws, nb, None)


def _bwd(lib, X=FAKE, dY=FAKE, T=4, q=None, A=FAKE, Bm=FAKE, r=8, alpha=16.0, U=None, dX=FAKE, dA=FAKE, dB=FAKE,
         ws=FAKE, nb=1 << 30):
    q = q if q is not None else _nf4(64, 64)
    return lib.qlora_linear_bwd(X, dY, T, ctypes.byref(q), A, Bm, r, alpha, U, dX, dA, dB, ws, nb, None)


def test_error_paths_forward(lib):
    E = B.QLORA_EINVAL
    assert _fwd(lib, X=None) == E
    assert _fwd(lib, Y=None) == E
    assert _fwd(lib, A=None) == E
    assert _fwd(lib, Bm=None) == E
    assert _fwd(lib, r=0) == E
    assert _fwd(lib, r=129) == E
    assert _fwd(lib, T=-1) == E
    assert _fwd(lib, alpha=float("inf")) == E
    assert _fwd(lib, X=MIS) == E
    assert _fwd(lib, U=MIS) == E
    assert _fwd(lib, q=_nf4(64, 100)) == E
    assert _fwd(lib, q=_nf4(60, 64)) == E  # n_out must be a multiple of 8 for the GEMMs
    assert _fwd(lib, ws=MIS) == E
    need = B.workspace_bytes(B.OP_FWD, 4, 64, 64, 8)
    assert _fwd(lib, nb=need - 1) == B.QLORA_EWORKSPACE
    assert "workspace" in lib.qlora_last_error().decode()


def test_error_paths_backward(lib):
    E = B.QLORA_EINVAL
    assert _bwd(lib, dA=None) == E
    assert _bwd(lib, dB=None) == E
    assert _bwd(lib, dY=None) == E
    assert _bwd(lib, X=None) == E
    assert _bwd(lib, dX=MIS) == E
    assert _bwd(lib, U=MIS) == E
    assert _bwd(lib, r=200) == E
    need = B.workspace_bytes(B.OP_BWD, 4, 64, 64, 8)
    assert _bwd(lib, nb=need - 1) == B.QLORA_EWORKSPACE


def _fwd_drop(lib, X=FAKE, T=4, q=None, A=FAKE, Bm=FAKE, r=8, alpha=16.0, p=0.05, seed=1, offset=0, mask=FAKE,
              Y=FAKE, U=None, ws=FAKE, nb=1 << 30):
    q = q if q is not None else _nf4(64, 64)
    return lib.qlora_linear_fwd_dropout(X, T, ctypes.byref(q), A, Bm, r, alpha, p, seed, offset, mask, Y, U, ws, nb,
                                        None)


def _bwd_drop(lib, X=FAKE, dY=FAKE, T=4, q=None, A=FAKE, Bm=FAKE, r=8, alpha=16.0, p=0.05, mask=FAKE, U=None,
              dX=FAKE, dA=FAKE, dB=FAKE, ws=FAKE, nb=1 << 30):
    q = q if q is not None else _nf4(64, 64)
    return lib.qlora_linear_bwd_dropout(X, dY, T, ctypes.byref(q), A, Bm, r, alpha, p, mask, U, dX, dA, dB, ws, nb,
                                        None)


def test_error_paths_dropout(lib):
    E = B.QLORA_EINVAL
    for bad_p in (-0.1, 1.0, 1.5, float("nan")):
        rc, msg = _err(lambda: _fwd_drop(lib, p=bad_p))
        assert rc == E and "probability" in msg, (bad_p, msg)
        assert _bwd_drop(lib, p=bad_p) == E
    rc, msg = _err(lambda: _fwd_drop(lib, mask=None))
    assert rc == E and "mask" in msg
    assert _bwd_drop(lib, mask=None) == E
    assert _fwd_drop(lib, mask=MIS) == E
    assert _bwd_drop(lib, mask=MIS) == E
    # the plain argument checks still apply
    assert _fwd_drop(lib, X=None) == E
    assert _bwd_drop(lib, dA=None) == E
    need = B.workspace_bytes(B.OP_FWD_DROPOUT, 4, 64, 64, 8)
    assert _fwd_drop(lib, nb=need - 1) == B.QLORA_EWORKSPACE
    need = B.workspace_bytes(B.OP_BWD, 4, 64, 64, 8)
    assert _bwd_drop(lib, nb=need - 1) == B.QLORA_EWORKSPACE


def test_dropout_workspace_covers_the_skinny_path(lib):
    """Few tokens take the GEMV path without dropout; with dropout the forward needs the split-K U pass."""
    for T in (1, 16, 64, 65, 2048):
        wd = B.workspace_bytes(B.OP_FWD_DROPOUT, T, 4096, 4096, 16)
        assert wd > 0
        if T > 64:
            assert wd == B.workspace_bytes(B.OP_FWD, T, 4096, 4096, 16)


def _adam(lib, descs, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0, step=1, count=None):
    arr = (B._AdamTensor * max(1, len(descs)))(*descs)
    return lib.qlora_adamw_step(arr, len(descs) if count is None else count, lr, b1, b2, eps, wd, step, None)


def test_error_paths_adamw(lib):
    E = B.QLORA_EINVAL
    ok = B._AdamTensor(0x1000, 0x2000, 0x3000, 0x4000, None, 100)
    assert _adam(lib, [ok], step=0) == E
    assert _adam(lib, [ok], b1=1.0) == E
    assert _adam(lib, [ok], b2=-0.1) == E
    assert _adam(lib, [ok], eps=0.0) == E
    assert _adam(lib, [ok], lr=-1.0) == E
    assert _adam(lib, [ok], wd=float("nan")) == E
    assert _adam(lib, [ok], count=-1) == E
    assert lib.qlora_adamw_step(None, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None) == E
    assert _adam(lib, [B._AdamTensor(0x1000, None, 0x3000, 0x4000, None, 100)]) == E
    assert _adam(lib, [B._AdamTensor(0x1008, 0x2000, 0x3000, 0x4000, None, 100)]) == E
    assert _adam(lib, [B._AdamTensor(0x1000, 0x2000, 0x3000, 0x4000, 0x5004, 100)]) == E
    assert _adam(lib, [B._AdamTensor(0x1000, 0x2000, 0x3000, 0x4000, None, -1)]) == E
    assert "tensor 1" in (_adam(lib, [ok, B._AdamTensor(0, 0, 0, 0, None, 5)]) == E and
                          lib.qlora_last_error().decode())
    # empty lists and empty tensors are fine without touching the device
    assert _adam(lib, []) == B.QLORA_OK


def test_error_paths_merge(lib):
    E = B.QLORA_EINVAL
    q = _nf4(64, 128)

    def merge(q_=q, Wb=None, n_out=64, n_in=128, A=FAKE, Bm=FAKE, r=8, alpha=16.0, W=FAKE, W32=None):
        return lib.qlora_merge(ctypes.byref(q_) if q_ is not None else None, Wb, n_out, n_in, A, Bm, r, alpha, W, W32,
                               None)

    rc, msg = _err(lambda: merge(Wb=FAKE))
    assert rc == E and "exactly one" in msg
    assert merge(q_=None) == E
    assert merge(n_out=32) == E  # shape differs from q
    assert merge(q_=None, Wb=FAKE, n_in=100) == E
    assert merge(q_=None, Wb=MIS) == E
    assert merge(r=0) == E and merge(r=129) == E
    assert merge(A=None) == E and merge(Bm=MIS) == E
    assert merge(W=None, W32=None) == E
    assert merge(W=MIS) == E
    assert merge(alpha=float("nan")) == E


def test_error_paths_multi(lib):
    E = B.QLORA_EINVAL
    q = _nf4(64, 128)

    def multi(X=FAKE, T=4, Ap=FAKE, Bp=FAKE, n_pool=3, r=8, alpha=16.0, seg=FAKE, ad=FAKE, n_seg=2, Y=FAKE, ws=FAKE,
              nb=1 << 30):
        return lib.qlora_linear_fwd_multi(X, T, ctypes.byref(q), Ap, Bp, n_pool, r, alpha, seg, ad, n_seg, Y, ws, nb,
                                          None)

    rc, msg = _err(lambda: multi(r=12))
    assert rc == E and "multiple of 8" in msg
    assert multi(n_pool=0) == E
    assert multi(n_seg=0) == E
    assert multi(seg=None) == E and multi(ad=None) == E
    assert multi(seg=ctypes.c_void_p(0x10002)) == E
    assert multi(Ap=None) == E and multi(Y=None) == E
    need = B.workspace_bytes(B.OP_FWD_MULTI, 4, 64, 128, 8)
    assert multi(nb=need - 1) == B.QLORA_EWORKSPACE


def test_error_paths_adamw8(lib):
    E = B.QLORA_EINVAL
    ok = B._Adam8Tensor(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, 100)

    def step(descs, **kw):
        arr = (B._Adam8Tensor * max(1, len(descs)))(*descs)
        args = dict(lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0, step=1)
        args.update(kw)
        return lib.qlora_adamw8_step(arr, len(descs), args["lr"], args["b1"], args["b2"], args["eps"], args["wd"],
                                     args["step"], None)

    assert step([ok], step=0) == E and step([ok], b1=1.0) == E and step([ok], eps=0.0) == E
    assert step([B._Adam8Tensor(0x1000, 0x2000, None, 0x4000, 0x5000, 0x6000, None, 100)]) == E
    assert step([B._Adam8Tensor(0x1000, 0x2000, 0x3008, 0x4000, 0x5000, 0x6000, None, 100)]) == E
    assert step([B._Adam8Tensor(0x1000, 0x2000, 0x3000, 0x4002, 0x5000, 0x6000, None, 100)]) == E
    assert step([]) == B.QLORA_OK
    if not gpu_available():
        assert step([ok]) == B.QLORA_ENODEV


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.qlora_strerror(code)
    assert lib.qlora_strerror(-99) == b"unknown error"


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path")
def test_no_device_is_reported(lib):
    """With valid-looking arguments and no GPU, the device check fails cleanly (no launch)."""
    q = _nf4(64, 64)
    assert lib.qlora_quantize_nf4(FAKE, ctypes.byref(q), None) == B.QLORA_ENODEV
    assert _fwd(lib) == B.QLORA_ENODEV
    assert _bwd(lib) == B.QLORA_ENODEV
    assert _fwd_drop(lib) == B.QLORA_ENODEV
    assert _bwd_drop(lib) == B.QLORA_ENODEV
    assert _adam(lib, [B._AdamTensor(0x1000, 0x2000, 0x3000, 0x4000, None, 100)]) == B.QLORA_ENODEV
    assert lib.qlora_merge(ctypes.byref(q), None, 64, 64, FAKE, FAKE, 8, 16.0, FAKE, None, None) == B.QLORA_ENODEV


def test_timing_api_host_only(lib):
    n, ms = B.timing_read("nf4_gemm_fwd")
    assert n == 0 and ms == 0.0
    B.timing_enable("nf4_gemm_fwd", True)
    B.timing_enable("nf4_gemm_fwd", False)
    assert lib.qlora_timing_enable(None, 1) == B.QLORA_EINVAL
    assert B.timing_read_each("nf4_gemm_fwd") == []
    n = ctypes.c_int64()
    assert lib.qlora_timing_read_each(b"nf4_gemm_fwd", None, 4, ctypes.byref(n)) == B.QLORA_EINVAL
    assert lib.qlora_timing_read_each(b"nf4_gemm_fwd", None, 0, None) == B.QLORA_EINVAL
