"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer and byte work (codes, 8-bit constants, steps, dequantized bf16 bits) must
match bit for bit.  Floating-point outputs (Y, U, dX, dA, dB) must satisfy, against
the binary64 oracle R:  ||G - R||_F / ||R||_F <= 1e-2  and
max |G - R| <= 3e-2 * max |R|.

Small and mid sizes are checked element by element in full; they span several
128x128 tiles and end in ragged tails (T, n_out not multiples of the tiles).
The full-size workloads are checked on 64 sampled token rows for Y and dX
(the oracle computes them one by one) and in full for dA and dB, plus adjoint
identities that hold at any size.
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_quantized_lora_02_amd import binding as Bd
from bit_quantized_lora_02_amd.synth import CONFIGS, linear_inputs

pytestmark = pytest.mark.gpu

REL_FRO = 1e-2
REL_MAX = 3e-2


def dev():
    return torch.device("cuda:0")


def to_gpu_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def gpu_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def gpu_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nref if nref > 0 else np.linalg.norm(got)
    mx = np.abs(got - ref).max() if got.size else 0.0
    bound = REL_MAX * np.abs(ref).max() if ref.size else 0.0
    assert rel <= REL_FRO, f"{name}: relative Frobenius error {rel:.3e} > {REL_FRO}"
    assert mx <= bound + (0.0 if nref > 0 else 1e-30), f"{name}: max abs error {mx:.3e} > {bound:.3e}"


def quantize_both(W: np.ndarray):
    n_out, n_in = W.shape
    w = Bd.quantize_nf4(torch.from_numpy(W).to(dev()))
    torch.cuda.synchronize()
    oc, oq, od = O.quantize_nf4(W)
    return w, (oc, oq, od)


# ------------------------------------------------------------ quantize / dequant

@pytest.mark.parametrize("shape,outliers", [((256, 256), 0.0), ((8, 64), 0.0), ((5, 4160), 0.0), ((72, 1152), 0.01),
                                            ((1024, 4096), 0.01)])
def test_quantize_and_dequant_bit_exact(shape, outliers):
    print(f"quantize {shape} outliers={outliers}", flush=True)
    inp = linear_inputs(shape[0], shape[1], 1, 4, 8.0, seed=1, outlier_frac=outliers, make_dy=False)
    W = inp.W
    W[0, :64] = 0.0  # an all-zero block
    W[0, 64:128] *= np.float32(1e-30)  # tiny constants (denormal products on decode)
    W[-1, 5] = -0.0
    w, (oc, oq, od) = quantize_both(W)
    np.testing.assert_array_equal(w.codes.cpu().numpy(), oc)
    np.testing.assert_array_equal(w.absmax_q.cpu().numpy(), oq)
    np.testing.assert_array_equal(w.absmax_step.cpu().numpy().view(np.uint32), od.view(np.uint32))
    deq = gpu_bits(Bd.dequant(w))
    np.testing.assert_array_equal(deq, O.dequant(oc, oq, od, *shape))


def test_quantize_ties_and_special_values():
    lv = O.nf4_levels()
    W = np.zeros((8, 128), np.float32)
    W[0, 0] = 1.0
    # exact midpoints that are binary32 values: the lower code wins
    mids = [(lv[i].astype(np.float64) + lv[i + 1]) / 2 for i in range(15)]
    k = 1
    for m in mids:
        if float(np.float32(m)) == m:
            W[0, k] = np.float32(m)
            W[0, k + 1] = np.nextafter(np.float32(m), np.float32(2))
            W[0, k + 2] = np.nextafter(np.float32(m), np.float32(-2))
            k += 3
    W[1, :64] = np.float32(-3.0)
    W[1, 0] = 3.0
    W[2, :] = lv[np.arange(128) % 16] * np.float32(0.25)
    W[3, 64:] = np.float32(2.0 ** -140)  # denormal weights
    w, (oc, oq, od) = quantize_both(W)
    np.testing.assert_array_equal(w.codes.cpu().numpy(), oc)
    np.testing.assert_array_equal(w.absmax_q.cpu().numpy(), oq)
    np.testing.assert_array_equal(w.absmax_step.cpu().numpy().view(np.uint32), od.view(np.uint32))
    np.testing.assert_array_equal(gpu_bits(Bd.dequant(w)), O.dequant(oc, oq, od, 8, 128))


def test_requantize_is_deterministic():
    inp = linear_inputs(512, 1024, 1, 4, 8.0, seed=2, make_dy=False)
    Wg = torch.from_numpy(inp.W).to(dev())
    a = Bd.quantize_nf4(Wg)
    b = Bd.quantize_nf4(Wg)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.absmax_q, b.absmax_q)
    assert torch.equal(a.absmax_step, b.absmax_step)


# ---------------------------------------------------------- forward / backward

def run_gpu(inp, w=None, need_dx=True, with_u=True):
    if w is None:
        w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    X, A, B, dY = (to_gpu_bf16(a) for a in (inp.X, inp.A, inp.B, inp.dY))
    Y, U = Bd.linear_fwd(X, w, A, B, inp.alpha, save_u=True)
    dX, dA, dB = Bd.linear_bwd(X, dY, w, A, B, inp.alpha, U=U if with_u else None, need_dx=need_dx)
    torch.cuda.synchronize()
    return w, dict(Y=Y, U=U, dX=dX, dA=dA, dB=dB)


def run_oracle(inp, rows=None):
    oc, oq, od = O.quantize_nf4(inp.W)
    Wd = O.dequant(oc, oq, od, *inp.W.shape)
    Y, U = O.linear_fwd(inp.X, Wd, inp.A, inp.B, inp.alpha, rows=rows)
    dX, dA, dB = O.linear_bwd(inp.X, inp.dY, Wd, inp.A, inp.B, inp.alpha, rows=rows)
    return dict(Y=Y, U=U, dX=dX, dA=dA, dB=dB)


SMALL = [
    # n_out, n_in, T, r, alpha
    (256, 256, 16, 8, 16.0),     # the CPU-sized workload
    (392, 320, 200, 16, 32.0),   # ragged tails in T and n_out, 2x3 tiles
    (136, 640, 131, 5, 7.0),     # odd rank, r not a multiple of anything
    (512, 192, 257, 64, 16.0),   # n_in with a half tile in dX
    (64, 128, 1, 128, 256.0),    # one token, maximum rank
    (1032, 256, 33, 12, 24.0),
    (72, 384, 20, 4, 8.0),       # 17..32 tokens through the small-token kernel, n_out not a multiple of 64
    (520, 192, 40, 8, 16.0),     # few tokens but n_in % 128 != 0: the tiled kernel
]


@pytest.mark.parametrize("n_out,n_in,T,r,alpha", SMALL)
def test_fwd_bwd_full_parity(n_out, n_in, T, r, alpha):
    print(f"parity n_out={n_out} n_in={n_in} T={T} r={r}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, alpha, seed=T + r)
    _, g = run_gpu(inp)
    ref = run_oracle(inp)
    for k in ("Y", "U", "dX", "dA", "dB"):
        assert_close(k, gpu_f64(g[k]), ref[k])
    # the backward without a saved U recomputes it and must agree bit for bit
    _, g2 = run_gpu(inp, with_u=False)
    for k in ("dX", "dA", "dB"):
        assert torch.equal(g[k], g2[k]), k


TRAINING_TILES = [
    # n_out, n_in, T, r, alpha: at least 256 output tiles of 256 x 256 (the largest tile), ragged in rows and
    # columns, with short reductions so that the whole oracle stays cheap; one to five 64-deep steps cover
    # the two-step loop and its tail
    (4104, 64, 4000, 5, 10.0),      # odd rank through the padded B
    (4096, 128, 4096, 128, 256.0),  # rank 128: two LoRA steps
    (4160, 192, 3900, 16, 32.0),
    (4104, 256, 4001, 64, 16.0),
    (4096, 320, 4096, 8, 16.0),
]


@pytest.mark.parametrize("n_out,n_in,T,r,alpha", TRAINING_TILES)
def test_training_tile_counts_full_parity(n_out, n_in, T, r, alpha):
    """Forward and backward at training-sized tile counts, checked in full against the oracle."""
    print(f"training-tile parity n_out={n_out} n_in={n_in} T={T} r={r}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, alpha, seed=T + n_in)
    _, g = run_gpu(inp)
    ref = run_oracle(inp)
    for k in ("Y", "U", "dX", "dA", "dB"):
        assert_close(k, gpu_f64(g[k]), ref[k])
    _, g2 = run_gpu(inp)  # bitwise repeatable
    assert torch.equal(g["Y"], g2["Y"]) and torch.equal(g["dX"], g2["dX"])


WHOLE_REDUCTION = [
    # n_out, n_in, T, r, alpha: >= 1024 tokens with r <= 16, where U and dU reduce inside one workgroup
    # (8-row tiles while they number at most the 256 CUs, else 16-row tiles)
    (1000, 192, 1031, 5, 10.0),   # n_in / 16 waves < 32: waves 6..15 get empty ranges; ragged 16-row tile
    (264, 640, 1024, 16, 32.0),   # exactly 64 row tiles
    (136, 1088, 1100, 1, 2.0),    # rank 1 (B through its zero-padded copy), reduction tail in every wave
    (72, 128, 2056, 12, 24.0),    # more 8-row tiles than CUs: 16-row tiles, the last one ragged
    (4104, 1088, 40, 16, 32.0),   # few tokens: U and dU split; n_out 4104 and n_in 1088 for dB and dA
]


SPLIT_FORWARD = [
    # n_out, n_in, T, r, alpha: more than 64 tokens but too few output tiles to occupy every CU, so the
    # forward GEMM splits its reduction into ranges (binary32 partial sums, added in order by a finalize)
    (1024, 2048, 128, 16, 32.0),  # 8 tiles, 32 steps: 4 ranges
    (520, 1024, 100, 128, 16.0),  # ragged tokens and rows, rank 128 (two LoRA steps in range 0): 2 ranges
    # at most 128 tokens over 96 or more 128x256 tiles take that tile: the forward here (2 ranges), the
    # backward's dX with n_in 24576 below
    (24576, 2048, 120, 16, 32.0),
    (512, 24576, 100, 8, 16.0),
]


@pytest.mark.parametrize("n_out,n_in,T,r,alpha", SPLIT_FORWARD)
def test_split_forward_parity(n_out, n_in, T, r, alpha):
    """The split-reduction forward GEMM, checked in full (and the backward of the same inputs)."""
    print(f"split forward parity n_out={n_out} n_in={n_in} T={T} r={r}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, alpha, seed=T + r)
    _, g = run_gpu(inp)
    ref = run_oracle(inp)
    for k in ("Y", "U", "dX", "dA", "dB"):
        assert_close(k, gpu_f64(g[k]), ref[k])
    _, g2 = run_gpu(inp)  # the same inputs again: bitwise repeatable
    assert torch.equal(g["Y"], g2["Y"])


@pytest.mark.parametrize("n_out,n_in,T,r,alpha", WHOLE_REDUCTION)
def test_whole_reduction_lora_parity(n_out, n_in, T, r, alpha):
    """U (forward and the backward's recompute) and dU through the whole-reduction kernel, checked in full."""
    print(f"whole-reduction parity n_out={n_out} n_in={n_in} T={T} r={r}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, alpha, seed=T + 7 * r)
    _, g = run_gpu(inp)
    ref = run_oracle(inp)
    for k in ("Y", "U", "dX", "dA", "dB"):
        assert_close(k, gpu_f64(g[k]), ref[k])
    _, g2 = run_gpu(inp, with_u=False)
    for k in ("dX", "dA", "dB"):
        assert torch.equal(g[k], g2[k]), k


def test_lora_dominated_parity():
    """Large adapters so the LoRA terms dominate every output (a dropped or
    mis-scaled LoRA term cannot hide under the base term's tolerance)."""
    inp = linear_inputs(264, 384, 77, 16, 32.0, seed=7, sigma_ab=0.5)
    _, g = run_gpu(inp)
    ref = run_oracle(inp)
    for k in ("Y", "U", "dX", "dA", "dB"):
        assert_close(k, gpu_f64(g[k]), ref[k])


def test_zero_weight_pure_lora():
    inp = linear_inputs(200, 256, 45, 8, 16.0, seed=8)
    inp.W[:] = 0.0
    _, g = run_gpu(inp)
    ref = run_oracle(inp)
    for k in ("Y", "dX", "dA", "dB"):
        assert_close(k, gpu_f64(g[k]), ref[k])
    assert float(g["Y"].float().abs().max()) > 0


def test_zero_adapter_cases():
    """B = 0: Y and dX equal the base terms and dA is exactly zero; A = 0: dB exactly zero."""
    inp = linear_inputs(264, 256, 70, 8, 16.0, seed=9)
    w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    zB = linear_inputs(264, 256, 70, 8, 16.0, seed=9)
    zB.B[:] = 0
    zA = linear_inputs(264, 256, 70, 8, 16.0, seed=9)
    zA.A[:] = 0
    _, gb = run_gpu(zB, w=w)
    _, ga = run_gpu(zA, w=w)
    assert torch.all(gb["dA"] == 0)
    assert torch.all(ga["dB"] == 0)
    # both reduce to X W'^T; only the sign of an exact zero may differ
    assert torch.equal(gb["Y"].float(), ga["Y"].float())
    ref = run_oracle(zB)
    assert_close("Y", gpu_f64(gb["Y"]), ref["Y"])
    assert_close("dX", gpu_f64(gb["dX"]), ref["dX"])


def test_empty_batch():
    inp = linear_inputs(64, 128, 0, 8, 16.0, seed=1)
    w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    X = torch.empty((0, 128), dtype=torch.bfloat16, device=dev())
    A, B = to_gpu_bf16(inp.A), to_gpu_bf16(inp.B)
    Y, U = Bd.linear_fwd(X, w, A, B, 16.0)
    assert Y.shape == (0, 64)
    dY = torch.empty((0, 64), dtype=torch.bfloat16, device=dev())
    dA = torch.full_like(A, 3.0)
    dB = torch.full_like(B, 3.0)
    dX = torch.empty_like(X)
    Bd.linear_bwd(X, dY, w, A, B, 16.0, outs=(dX, dA, dB))
    torch.cuda.synchronize()
    assert torch.all(dA == 0) and torch.all(dB == 0)


def test_repeatable_and_weight_frozen():
    inp = linear_inputs(520, 512, 300, 16, 32.0, seed=10)
    w, g1 = run_gpu(inp)
    before = (w.codes.clone(), w.absmax_q.clone(), w.absmax_step.clone())
    _, g2 = run_gpu(inp, w=w)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
    assert torch.equal(before[0], w.codes) and torch.equal(before[1], w.absmax_q)
    assert torch.equal(before[2], w.absmax_step)


@pytest.mark.parametrize("n_out,n_in,T", [(1032, 4096, 1), (1000, 4096, 8), (1032, 2048, 40), (520, 1536, 17)])
def test_few_token_forward_is_bitwise_repeatable(n_out, n_in, T):
    """The few-token kernels add their split partial sums in a fixed order (no atomics): the same call on the
    same inputs gives the same bits, whatever the workspace held before (row kernel, 32-token kernel with one
    and two token groups, 16-row kernel)."""
    print(f"few-token repeatability {n_out}x{n_in} T={T}", flush=True)
    inp = linear_inputs(n_out, n_in, T, 16, 32.0, seed=n_out + T)
    w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    X, A, B = (to_gpu_bf16(a) for a in (inp.X, inp.A, inp.B))
    Y1, U1 = Bd.linear_fwd(X, w, A, B, inp.alpha)
    Y2, U2 = Bd.linear_fwd(X, w, A, B, inp.alpha)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(U1, U2)


def test_autograd_function():
    inp = linear_inputs(136, 192, 40, 8, 16.0, seed=12)
    w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    X = to_gpu_bf16(inp.X).requires_grad_(True)
    A = to_gpu_bf16(inp.A).requires_grad_(True)
    B = to_gpu_bf16(inp.B).requires_grad_(True)
    Y = Bd.QLoRALinearFn.apply(X, w, A, B, inp.alpha)
    Y.backward(to_gpu_bf16(inp.dY))
    ref = run_oracle(inp)
    assert_close("Y", gpu_f64(Y), ref["Y"])
    assert_close("dX", gpu_f64(X.grad), ref["dX"])
    assert_close("dA", gpu_f64(A.grad), ref["dA"])
    assert_close("dB", gpu_f64(B.grad), ref["dB"])


@pytest.mark.parametrize("T,kernel", [(200, "nf4_gemm_fwd"), (8, "nf4_gemv")])
def test_timing_hook_counts_launches(T, kernel):
    inp = linear_inputs(256, 256, T, 8, 16.0, seed=13)
    w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    Bd.timing_enable(kernel, True)
    for _ in range(3):
        run_gpu(inp, w=w)
    Bd.timing_enable(kernel, False)
    n, ms = Bd.timing_read(kernel)
    assert n == 3 and ms > 0


# ------------------------------------------------------------- full sizes

def _full_size_cases():
    out = []
    for cfg in ("attn_4096", "mlp_8b", "layer_70b"):
        c = CONFIGS[cfg]
        for name, n_out, n_in in c["linears"]:
            out.append(pytest.param(cfg, name, n_out, n_in, c["T"], c["r"], c["alpha"], c["outliers"],
                                    id=f"{cfg}-{name}"))
    return out


@pytest.mark.parametrize("cfg,name,n_out,n_in,T,r,alpha,outliers", _full_size_cases())
def test_full_size_sampled(cfg, name, n_out, n_in, T, r, alpha, outliers):
    print(f"full size {cfg}/{name}: {n_out}x{n_in} T={T} r={r}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, alpha, seed=0, outlier_frac=outliers)
    w, g = run_gpu(inp)
    oc, oq, od = O.quantize_nf4(inp.W)
    assert np.array_equal(w.codes.cpu().numpy(), oc)
    assert np.array_equal(w.absmax_q.cpu().numpy(), oq)
    assert np.array_equal(w.absmax_step.cpu().numpy().view(np.uint32), od.view(np.uint32))
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(1).choice(T, 62, replace=False)]))
    ref = run_oracle(inp, rows=rows)
    idx = torch.from_numpy(rows).to(dev())
    assert_close("Y", gpu_f64(g["Y"][idx]), ref["Y"])
    assert_close("U", gpu_f64(g["U"][idx]), ref["U"])
    assert_close("dX", gpu_f64(g["dX"][idx]), ref["dX"])
    assert_close("dA", gpu_f64(g["dA"]), ref["dA"])
    assert_close("dB", gpu_f64(g["dB"]), ref["dB"])
    # adjoint identities over the whole outputs: <dX, X> = <dY, Y>, <dA, A> = <dB, B>
    X, dY, A, B = (O.bf16_bits_to_f64(a) for a in (inp.X, inp.dY, inp.A, inp.B))
    lhs, rhs = np.sum(gpu_f64(g["dX"]) * X), np.sum(dY * gpu_f64(g["Y"]))
    assert abs(lhs - rhs) <= 1e-2 * np.sqrt(np.sum(gpu_f64(g["dX"]) ** 2) * np.sum(X ** 2))
    la, lb = np.sum(gpu_f64(g["dA"]) * A), np.sum(gpu_f64(g["dB"]) * B)
    assert abs(la - lb) <= 1e-2 * max(abs(la), abs(lb))


@pytest.mark.parametrize("n_out,n_in,T,r", [(4104, 4096, 4133, 16), (1032, 2048, 8200, 40), (1024, 8192, 1024, 16),
                                            (2000, 8192, 2000, 8)])
def test_large_ragged_sampled(n_out, n_in, T, r):
    """Shapes large enough for the 256-row tiles, with partial tiles in T and n_out.  The last two are narrow
    outputs of many tokens, whose forward takes 256x256 tiles with the reduction split in 16 and 4 ranges
    (the second ragged in T and n_out)."""
    print(f"large ragged {n_out}x{n_in} T={T} r={r}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, 2.0 * r, seed=3)
    _, g = run_gpu(inp)
    rows = np.unique(np.concatenate([[0, T - 1, T - 2], np.random.default_rng(2).choice(T, 40, replace=False)]))
    ref = run_oracle(inp, rows=rows)
    idx = torch.from_numpy(rows).to(dev())
    for k in ("Y", "U", "dX"):
        assert_close(k, gpu_f64(g[k][idx]), ref[k])
    assert_close("dA", gpu_f64(g["dA"]), ref["dA"])
    assert_close("dB", gpu_f64(g["dB"]), ref["dB"])


@pytest.mark.parametrize("n_out", [8192, 28672])
@pytest.mark.parametrize("T", [1, 8, 32, 128])
def test_small_token_forward(n_out, T):
    print(f"small-token forward {n_out}x8192 T={T}", flush=True)
    c = CONFIGS["small_token"]
    inp = linear_inputs(n_out, 8192, T, c["r"], c["alpha"], seed=0)
    w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    X, A, B = (to_gpu_bf16(a) for a in (inp.X, inp.A, inp.B))
    Y, U = Bd.linear_fwd(X, w, A, B, inp.alpha)
    torch.cuda.synchronize()
    oc, oq, od = O.quantize_nf4(inp.W)
    Wd = O.dequant(oc, oq, od, n_out, 8192)
    rows = np.arange(T) if T <= 8 else np.unique(np.concatenate([[0, T - 1], np.arange(1, T, T // 8)]))
    Yr, Ur = O.linear_fwd(inp.X, Wd, inp.A, inp.B, inp.alpha, rows=rows)
    idx = torch.from_numpy(rows).to(dev())
    assert_close("Y", gpu_f64(Y[idx]), Yr)
    assert_close("U", gpu_f64(U[idx]), Ur)


@pytest.mark.parametrize("n_out,n_in,T,r", [(72, 512, 3, 16), (8, 1536, 16, 4), (1000, 4096, 9, 1),
                                            (24, 8192, 16, 64), (136, 8704, 5, 8), (72, 512, 32, 16),
                                            (8, 8192, 24, 8), (520, 1536, 17, 4), (24, 8448, 20, 8),
                                            (136, 1024, 19, 16), (40, 3072, 32, 8), (1000, 2048, 25, 16),
                                            (24, 28672, 8, 8), (40, 16384, 20, 4), (8, 32768, 32, 8),
                                            (8, 65536, 4, 8), (8, 66560, 4, 8), (8, 33024, 24, 4),
                                            (72, 1024, 33, 16), (136, 8192, 64, 8), (40, 1152, 48, 4),
                                            (8, 16384, 64, 4), (8, 16512, 40, 4), (40, 1536, 40, 8),
                                            (8, 32768, 36, 4)])
def test_row_group_forward(n_out, n_in, T, r):
    """3..64 tokens through the row-group kernels.  Where n_in is a multiple of 2048 (up to 32 tokens) or 1024
    (33-64) with at most 32 parts, the 32-token kernel takes the shape (4096, 8192, 2048, 28672, 16384, 32768
    up to 32 tokens; 1024, 8192, 16384, 32768 beyond); the rest keep the 16-row kernel (16 rows per wave,
    activations in registers, exactly dequantized weights), described next: one token
    group and segments of 512 columns up to 16 tokens, two groups and segments of 256 up to 32, four groups
    and segments of 128 beyond, only when the segments come in fours (1152 and 16512: 9 and 129 segments,
    the MFMA kernel).  With two or four token groups and a segment count divisible by 8 the eight waves of a
    workgroup add their segments before writing (n_in 1024, 8192, 16384 and 32768 at 33-64 tokens: 1, 8,
    16 and 32 partials; 2048, 8192, 16384 and 32768 at 17-32); otherwise, with a count divisible by 4, the
    four waves of a workgroup do (n_in 1536 at 40 tokens, 1024 and 3072 at 17-32, 4096 .. 65536 up to 16
    tokens: 1 to 32 partials); otherwise each segment is a partial (n_in 512, 1536, 8704: 1 to 17).  At most 32
    partials reach the finish kernel; the shapes past that (8448 and 33024 at 20-24 tokens, 66560 at 4)
    take the MFMA kernel; checked in full."""
    print(f"row-group forward {n_out}x{n_in} T={T} r={r}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, 2.0 * r, seed=n_out + 3 * T, sigma_ab=0.05)
    w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    X, A, B = (to_gpu_bf16(a) for a in (inp.X, inp.A, inp.B))
    Y, U = Bd.linear_fwd(X, w, A, B, inp.alpha)
    torch.cuda.synchronize()
    oc, oq, od = O.quantize_nf4(inp.W)
    Yr, Ur = O.linear_fwd(inp.X, O.dequant(oc, oq, od, n_out, n_in), inp.A, inp.B, inp.alpha)
    assert_close("Y", gpu_f64(Y), Yr)
    assert_close("U", gpu_f64(U), Ur)


@pytest.mark.parametrize("n_out,n_in,T,r", [(72, 2048, 3, 16), (1000, 8192, 32, 16), (2056, 8192, 32, 16),
                                            (200, 28672, 17, 64), (4104, 2048, 8, 16), (8, 65536, 32, 8),
                                            (520, 4096, 12, 128), (24, 6144, 24, 4), (1032, 2048, 9, 1),
                                            (40, 14336, 31, 16), (1000, 8192, 64, 16), (200, 28672, 33, 64),
                                            (2056, 4096, 40, 16), (24, 1024, 57, 128), (8, 32768, 48, 8)])
def test_32_token_row_group_forward(n_out, n_in, T, r):
    """3..64 tokens with n_in a multiple of 2048 (up to 32 tokens) or 1024 (33-64): the 32-token row-group
    kernel (32x32x16 MFMAs, tokens as M in one or two groups of 32, the block constant applied to each block's
    MFMA result, eight segments of 256 or 128 columns per workgroup added through LDS: 1 to 32 partials),
    including ragged row groups (n_out 1000, 200, 520, 24, 40, 8), several items per workgroup (2056 and 4104
    rows), the last token of each 8-token group (T 8, 24, 32, 40, 48, 64) and one past it (9, 17, 33, 57),
    rank 128 and rank 1; checked in full."""
    print(f"32-token row-group forward {n_out}x{n_in} T={T} r={r}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, 2.0 * r, seed=n_out + 5 * T, sigma_ab=0.05)
    w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    X, A, B = (to_gpu_bf16(a) for a in (inp.X, inp.A, inp.B))
    Y, U = Bd.linear_fwd(X, w, A, B, inp.alpha)
    torch.cuda.synchronize()
    oc, oq, od = O.quantize_nf4(inp.W)
    Yr, Ur = O.linear_fwd(inp.X, O.dequant(oc, oq, od, n_out, n_in), inp.A, inp.B, inp.alpha)
    assert_close("Y", gpu_f64(Y), Yr)
    assert_close("U", gpu_f64(U), Ur)


@pytest.mark.parametrize("n_out,n_in,T,r", [(72, 2048, 1, 16), (1032, 4096, 2, 5), (520, 8192, 1, 32),
                                            (264, 16384, 2, 64), (8, 2048, 2, 8), (4104, 6144, 1, 12),
                                            (2056, 4096, 2, 24), (6152, 8192, 1, 16), (520, 8192, 3, 16),
                                            (8, 2048, 4, 8), (8, 2048, 1, 1), (16, 4096, 2, 3),
                                            (8, 65536, 1, 8), (24, 32768, 2, 4), (8, 34816, 1, 8)])
def test_row_streaming_forward(n_out, n_in, T, r):
    """Few tokens with n_in % 2048 == 0: the row-streaming kernel (1-2 tokens, one wave per weight row, rows cut
    into segments of 4096 or 2048 columns, up to 16 of them: n_in 65536 with one token, 32768 with two) and the
    MFMA kernel (3-4 tokens, or 17 segments: n_in 34816), checked in full."""
    print(f"row-streaming forward {n_out}x{n_in} T={T} r={r}", flush=True)
    inp = linear_inputs(n_out, n_in, T, r, 2.0 * r, seed=n_out + T, sigma_ab=0.05)
    w = Bd.quantize_nf4(torch.from_numpy(inp.W).to(dev()))
    X, A, B = (to_gpu_bf16(a) for a in (inp.X, inp.A, inp.B))
    Y, U = Bd.linear_fwd(X, w, A, B, inp.alpha)
    torch.cuda.synchronize()
    oc, oq, od = O.quantize_nf4(inp.W)
    Yr, Ur = O.linear_fwd(inp.X, O.dequant(oc, oq, od, n_out, n_in), inp.A, inp.B, inp.alpha)
    assert_close("Y", gpu_f64(Y), Yr)
    assert_close("U", gpu_f64(U), Ur)
