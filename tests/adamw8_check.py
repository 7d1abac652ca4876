"""Judge one 8-bit AdamW step taken in binary32 against the binary64 step of the oracle.

Test helper (not a test module).  The binary64 step (oracle.adamw8_step_f64) decodes the
moments exactly, takes the binary64 AdamW and encodes by exact midpoints.  A binary32 step
from the same state differs from it only by the roundings of its own arithmetic; the bounds
below follow each of those roundings (unit roundoff u = 2^-24 per binary32 operation, every
constant rounded once from binary64), doubled for margin:

  new first moment    b1 m + (1 - b1) g:   4u (|b1 m| + |(1 - b1) g|) + u |m'|
  new second moment   b2 v + (1 - b2) g^2: 4u (b2 v + (1 - b2) g^2) + u v'
  block absmax        max |m'|: at most the largest moment error of its block
  x = m' / absmax     u |x| + (err + |x| err_absmax) / absmax
  parameter           3u |theta (1 - lr wd)| + (lr / bc1) err_m / d + 10u |update|,
                      d = sqrt(v' / bc2) + eps

A stored code must equal the binary64 code, or be its neighbour in the ordered book with the
midpoint between the two within the x bound of the binary64 value (the binary32 value fell on
the other side of it).  The block absmax must lie within its bound; the parameter (and the
master copy) within the parameter bound, the bf16 parameter within half a bf16 unit more.
"""
import numpy as np

U = 2.0 ** -24


def decode(book, codes, absmax):
    """Stored moments as binary64 (book value times block absmax: exact in binary64)."""
    ab = np.repeat(np.asarray(absmax, np.float64), 2048)[: codes.size]
    return book[codes].astype(np.float64) * ab


def _position(codes, signed):
    """Place of each code in the book ordered by value (signed book: -127 .. 127)."""
    c = codes.astype(np.int64)
    if not signed:
        return c
    mag = c & 127
    return np.where(c & 128, -mag, mag)


def _value_at(book, pos, signed):
    if not signed:
        return book[pos].astype(np.float64)
    mag = book[np.abs(pos)].astype(np.float64)
    return np.where(pos < 0, -mag, mag)


def _codes_ok(name, got, want, x64, tol, book, signed):
    pg, pw = _position(got, signed), _position(want, signed)
    diff = pg != pw
    if not diff.any():
        return 0
    idx = np.flatnonzero(diff)
    adj = np.abs(pg[idx] - pw[idx]) == 1
    lo = np.minimum(pg[idx], pw[idx])
    mid = 0.5 * (_value_at(book, lo, signed) + _value_at(book, lo + 1, signed))
    near = np.abs(mid - x64[idx]) <= tol[idx]
    bad = idx[~(adj & near)]
    assert bad.size == 0, (name, bad[:5], got[bad][:5], want[bad][:5], x64[bad][:5], tol[bad][:5])
    return idx.size


def check_step(got, ref, theta_in, g_bits, mo, vo, sbook, ubook, lr, b1, b2, eps, wd, t, bf16_to_f64):
    """got: the binary32 step's state after the step (mc, vc, ma, va as stored; p bf16 bits; master or
    None); ref: oracle.adamw8_step_f64 from the same state; theta_in, mo, vo: the parameter and the
    decoded moments before the step (binary64); g_bits the gradient.  Returns the number of code flips."""
    n = g_bits.size
    g = bf16_to_f64(g_bits).reshape(-1)
    m64, v64 = ref["m"], ref["v"]
    err_m = 2 * (4 * U * (np.abs(b1 * mo) + np.abs((1 - b1) * g)) + U * np.abs(m64))
    err_v = 2 * (4 * U * (b2 * vo + (1 - b2) * g * g) + U * v64)
    flips = 0
    for blk in range((n + 2047) // 2048):
        sl = slice(blk * 2048, min(n, (blk + 1) * 2048))
        for key, codes_key, book, signed, val, err in (("ma", "mc", sbook, True, m64, err_m),
                                                       ("va", "vc", ubook, False, v64, err_v)):
            am64 = ref[key][blk]
            emax = err[sl].max()
            am32 = float(got[key][blk])
            assert abs(am32 - am64) <= emax, (key, blk, am32, am64, emax)
            if am64 == 0.0:
                assert np.all(got[codes_key][sl] == 0), (codes_key, blk)
                continue
            x64 = val[sl] / am64
            tol = 2 * (U * np.abs(x64) + (err[sl] + np.abs(x64) * emax) / am64)
            flips += _codes_ok(codes_key, got[codes_key][sl], ref[codes_key][sl], x64, tol, book, signed)
    bc1, bc2 = 1.0 - b1 ** t, 1.0 - b2 ** t
    d = np.sqrt(v64 / bc2) + eps
    upd = (lr / bc1) * m64 / d
    err_th = 2 * (3 * U * np.abs(theta_in * (1 - lr * wd)) + (lr / bc1) * err_m / d + 10 * U * np.abs(upd))
    th64 = ref["theta"]
    if got.get("master") is not None:
        master = np.asarray(got["master"], np.float64).reshape(-1)
        bad = np.abs(master - th64) > err_th
        assert not bad.any(), ("master", np.flatnonzero(bad)[:5], master[bad][:5], th64[bad][:5])
    p = bf16_to_f64(got["p"]).reshape(-1)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(th64), 1e-38))) - 7)
    bad = np.abs(p - th64) > 0.5 * ulp + err_th
    assert not bad.any(), ("param", np.flatnonzero(bad)[:5], p[bad][:5], th64[bad][:5])
    return flips
