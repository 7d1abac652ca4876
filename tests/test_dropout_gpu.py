"""GPU parity of the LoRA-dropout path (through the C ABI) against the CPU oracle.

The keep-bit mask is integer work and must match the oracle's bit for bit; Y,
U, dX, dA and dB are held to the same bounds as the dropout-free path
(relative Frobenius error <= 1e-2, max abs error <= 3e-2 max |R|).  The
probability 0.05 is the one the pages configure ("Module 08 - QLoRA &
Quantization", "4. QLoRA in code"); 0.5 makes every output depend visibly on
the mask.
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_quantized_lora_02_amd import binding as Bd
from bit_quantized_lora_02_amd.synth import CONFIGS, linear_inputs
from test_parity_gpu import assert_close, dev, gpu_f64, to_gpu_bf16

pytestmark = pytest.mark.gpu


def run_gpu_drop(inp, p, seed, offset, w=None, with_u=True, need_dx=True):
    if w is None:
        w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    X, A, B, dY = (to_gpu_bf16(a) for a in (inp.X, inp.A, inp.B, inp.dY))
    Y, U, mask = Bd.linear_fwd_dropout(X, w, A, B, inp.alpha, p, seed, offset)
    dX, dA, dB = Bd.linear_bwd_dropout(X, dY, w, A, B, inp.alpha, p, mask, U=U if with_u else None,
                                       need_dx=need_dx)
    torch.cuda.synchronize()
    return w, dict(Y=Y, U=U, dX=dX, dA=dA, dB=dB, mask=mask)


def oracle_drop(inp, p, mask, rows=None):
    oc, oq, od = O.quantize_nf4(inp.W)
    Wd = O.dequant(oc, oq, od, *inp.W.shape)
    Y, U = O.linear_fwd_dropout(inp.X, Wd, inp.A, inp.B, inp.alpha, mask, p, rows=rows)
    dX, dA, dB = O.linear_bwd_dropout(inp.X, inp.dY, Wd, inp.A, inp.B, inp.alpha, mask, p, rows=rows)
    return dict(Y=Y, U=U, dX=dX, dA=dA, dB=dB)


CASES = [
    # n_out, n_in, T, r, alpha, p
    (256, 256, 16, 8, 16.0, 0.05),
    (392, 320, 200, 16, 32.0, 0.05),   # ragged T and n_out
    (136, 640, 131, 5, 7.0, 0.5),      # odd rank
    (512, 192, 257, 64, 16.0, 0.5),    # n_in with a half tile in dX
    (64, 128, 1, 128, 256.0, 0.05),    # one token, maximum rank
    (72, 384, 20, 4, 8.0, 0.3),        # few tokens: the dropout forward takes the tiled path
    (1032, 256, 33, 12, 24.0, 0.05),
]


@pytest.mark.parametrize("n_out,n_in,T,r,alpha,p", CASES)
def test_dropout_full_parity(n_out, n_in, T, r, alpha, p):
    print(f"dropout parity n_out={n_out} n_in={n_in} T={T} r={r} p={p}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, alpha, seed=100 + T + r, sigma_ab=0.2)
    seed, offset = 1234 + T, 5
    w, g = run_gpu_drop(inp, p, seed, offset)
    mask = O.dropout_mask(T, n_in, p, seed, offset)
    np.testing.assert_array_equal(g["mask"].cpu().numpy(), mask)
    ref = oracle_drop(inp, p, mask)
    for k in ("Y", "U", "dX", "dA", "dB"):
        assert_close(k, gpu_f64(g[k]), ref[k])
    # recomputing U from X and the mask gives the same gradients bit for bit
    _, g2 = run_gpu_drop(inp, p, seed, offset, w=w, with_u=False)
    for k in ("mask", "dX", "dA", "dB"):
        assert torch.equal(g[k], g2[k]), k


def test_dropout_mask_matters():
    """At p = 1/2 the outputs differ from the dropout-free ones and from another offset's."""
    inp = linear_inputs(264, 384, 77, 16, 32.0, seed=7, sigma_ab=0.5)
    w, g0 = run_gpu_drop(inp, 0.5, 9, 0)
    _, g1 = run_gpu_drop(inp, 0.5, 9, 1, w=w)
    assert not torch.equal(g0["mask"], g1["mask"])
    for k in ("Y", "dX", "dA"):
        assert not torch.equal(g0[k], g1[k]), k
    keep = np.unpackbits(g0["mask"].cpu().numpy()).mean()
    assert 0.45 < keep < 0.55
    ref = oracle_drop(inp, 0.5, g0["mask"].cpu().numpy())
    for k in ("Y", "U", "dX", "dA", "dB"):
        assert_close(k, gpu_f64(g0[k]), ref[k])


def test_dropout_p_zero_equals_plain_path():
    """p = 0 keeps every element with q = 1: Y, U, dA and dB are those of the dropout-free path bit for bit;
    dX (adapter term summed first) agrees with the oracle."""
    inp = linear_inputs(264, 256, 70, 8, 16.0, seed=9)
    w, g = run_gpu_drop(inp, 0.0, 3, 0)
    assert torch.all(g["mask"] == 0xFF)
    X, A, B, dY = (to_gpu_bf16(a) for a in (inp.X, inp.A, inp.B, inp.dY))
    Y, U = Bd.linear_fwd(X, w, A, B, inp.alpha)
    dX, dA, dB = Bd.linear_bwd(X, dY, w, A, B, inp.alpha, U=U)
    torch.cuda.synchronize()
    for k, v in (("Y", Y), ("U", U), ("dA", dA), ("dB", dB)):
        assert torch.equal(g[k], v), k
    oc, oq, od = O.quantize_nf4(inp.W)
    ref = O.linear_bwd(inp.X, inp.dY, O.dequant(oc, oq, od, 264, 256), inp.A, inp.B, inp.alpha)
    assert_close("dX", gpu_f64(g["dX"]), ref[0])


def test_dropout_repeatable():
    inp = linear_inputs(520, 512, 300, 16, 32.0, seed=10)
    w, g1 = run_gpu_drop(inp, 0.05, 77, 3)
    _, g2 = run_gpu_drop(inp, 0.05, 77, 3, w=w)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_dropout_empty_batch():
    inp = linear_inputs(64, 128, 0, 8, 16.0, seed=1)
    w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    X = torch.empty((0, 128), dtype=torch.bfloat16, device=dev())
    A, B = to_gpu_bf16(inp.A), to_gpu_bf16(inp.B)
    Y, U, mask = Bd.linear_fwd_dropout(X, w, A, B, 16.0, 0.05, 1)
    assert Y.shape == (0, 64) and mask.numel() == 0
    dY = torch.empty((0, 64), dtype=torch.bfloat16, device=dev())
    dA = torch.full_like(A, 3.0)
    dB = torch.full_like(B, 3.0)
    Bd.linear_bwd_dropout(X, dY, w, A, B, 16.0, 0.05, mask, outs=(torch.empty_like(X), dA, dB))
    torch.cuda.synchronize()
    assert torch.all(dA == 0) and torch.all(dB == 0)


def test_dropout_attention_size_sampled():
    """The attention workload (4096 x 4096, T = 2048, r = 16) at p = 0.05, in the launch configuration the
    benchmark times: the whole mask bit for bit, dA and dB in full, Y, U and dX on sampled rows."""
    c = CONFIGS["attn_4096"]
    _, n_out, n_in = c["linears"][0]
    T = c["T"]
    print(f"dropout full size {n_out}x{n_in} T={T}", flush=True)
    inp = linear_inputs(n_out, n_in, T, c["r"], c["alpha"], seed=0)
    _, g = run_gpu_drop(inp, 0.05, 2024, 11)
    mask = O.dropout_mask(T, n_in, 0.05, 2024, 11)
    np.testing.assert_array_equal(g["mask"].cpu().numpy(), mask)
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(4).choice(T, 30, replace=False)]))
    ref = oracle_drop(inp, 0.05, mask, rows=rows)
    idx = torch.from_numpy(rows).to(dev())
    for k in ("Y", "U", "dX"):
        assert_close(k, gpu_f64(g[k][idx]), ref[k])
    assert_close("dA", gpu_f64(g["dA"]), ref["dA"])
    assert_close("dB", gpu_f64(g["dB"]), ref["dB"])


def test_dropout_large_dx_tiles_sampled():
    """dX of 4096 x 4096 tokens x features: without dropout the 256x256 tile; with it the 256x128 tile with the
    per-tile adapter epilogue.  Mask bit for bit, dA and dB in full, dX, Y and U on sampled rows."""
    n_out, n_in, T, r = 1024, 4096, 4096, 16
    print(f"dropout large tiles {n_out}x{n_in} T={T}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, 32.0, seed=5, sigma_ab=0.1)
    _, g = run_gpu_drop(inp, 0.1, 77, 1)
    mask = O.dropout_mask(T, n_in, 0.1, 77, 1)
    np.testing.assert_array_equal(g["mask"].cpu().numpy(), mask)
    rows = np.unique(np.concatenate([[0, 255, 256, T - 1], np.random.default_rng(6).choice(T, 28, replace=False)]))
    ref = oracle_drop(inp, 0.1, mask, rows=rows)
    idx = torch.from_numpy(rows).to(dev())
    for k in ("Y", "U", "dX"):
        assert_close(k, gpu_f64(g[k][idx]), ref[k])
    assert_close("dA", gpu_f64(g["dA"]), ref["dA"])
    assert_close("dB", gpu_f64(g["dB"]), ref["dB"])
