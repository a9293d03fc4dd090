"""Parity of the W8A8 path (through the C ABI) with the CPU oracle.

The pages' second setting: 8-bit weights and activations (the lsdiaocha.cn write-up of the paper:
W8A8 next to W4A4), quantized as page "十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com),
训练后量化（PTQ）, defines the N-bit quantizer, here with N = 8: scale absmax / 127, codes in
[-128, 127].  The rotation and smoothing are those of the W4A4 path.  Acceptance is the W4A4 rule
set (tests/acceptance.py) with qmax = 127: int32 accumulators bit-exact on identical codes, codes
admissible and mismatched at <= 1e-4, outputs within 1e-3 (fp32) or one bf16 ulp.
"""
import numpy as np
import pytest

import acceptance as acc
from guard import check_codes_guard, check_guard, guarded_codes, guarded_output
import oracle
from bit_ptq_reconstruction_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

Q8 = 127


@pytest.fixture(scope="module")
def qv():
    import bit_ptq_reconstruction_amd as m

    m.lib()
    return m


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(a, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def run_quant8(qv, dev, X, dtype, mult, weights=False):
    M, K = X.shape
    qfull, q, sfull, s = guarded_codes(M, K, 0, dev, code_dtype=torch.int8, code_fill=0x55)
    md = None if mult is None else torch.from_numpy(mult).to(dev)
    (qv.qv_pack_weights8 if weights else qv.qv_hadamard_smooth_quant8)(to_dev(X, dtype, dev), md, q, s)
    torch.cuda.synchronize()
    check_codes_guard(qfull, sfull, M, code_fill=0x55, label=f"rotate-quantize8 M={M} K={K}")
    return q.cpu().numpy(), s.cpu().numpy()


def check_quant8(X, mult, q_gpu, s_gpu, label):
    Xhat = oracle.rotate(X, oracle.ROT_FWHT)
    q_ref, s_ref = oracle.quantize_rows(Xhat, mult, bits=8)
    t, tau, _, rel = acc.code_bounds(X, mult, Xhat, qmax=Q8)
    rate = acc.check_codes(q_gpu, q_ref, t, tau, label, qmax=Q8)
    acc.check_scales(s_gpu, s_ref, rel, label)
    return rate, np.where(q_gpu != q_ref, q_gpu, q_ref), s_ref


@pytest.mark.parametrize("K,dtype,M,smooth", [(1024, "fp32", 1, False), (1024, "bf16", 137, True),
                                              (4096, "bf16", 70, True), (4096, "fp32", 1375, False),
                                              (1024, "bf16", 1375, True)])
def test_quant8_parity(qv, dev, K, dtype, M, smooth):
    X = synth.vggt_activations(M, K, seed=M + K, dtype=dtype)
    mult = None
    if smooth:
        W = synth.weights(256, K, seed=3)
        _, mult = oracle.smoothing(oracle.rotate(X[:1374], oracle.ROT_FWHT), oracle.rotate(W, oracle.ROT_FWHT), 0.5)
    q, s = run_quant8(qv, dev, X, dtype, mult)
    rate, _, _ = check_quant8(X, mult, q, s, f"int8 K={K} {dtype} M={M}")
    print(f"int8 K={K} {dtype} M={M}: code mismatch rate {rate:.2e}")


@pytest.mark.parametrize("K", [1024, 4096])
def test_quant8_constructed_ties_and_special_rows(qv, dev, K):
    """Half-integer targets with max |t| = 127 rotate back exactly: scale 1, codes rint(t) bit-exact;
    zero and subnormal rows give scale 0 and zero codes; a one-hot row spreads to +-127."""
    rng = np.random.default_rng(K)
    t = rng.integers(-254, 255, size=(3, K)).astype(np.float64) / 2.0
    t[:, 0] = 127.0
    H = oracle.hadamard(K).astype(np.float64)
    X = (t @ H / np.sqrt(K)).astype(np.float32)
    assert np.array_equal(X.astype(np.float64) @ H.T / np.sqrt(K), t)  # exact in fp32
    Z = np.zeros((3, K), np.float32)
    Z[1, :] = 1e-41
    Z[2, 11] = 300.0
    q, s = run_quant8(qv, dev, np.concatenate([X, Z]), "fp32", None)
    np.testing.assert_array_equal(q[:3], np.rint(t).astype(np.int8))
    assert np.all(s[:3] == 1.0)
    assert s[3] == 0 and s[4] == 0 and np.all(q[3:5] == 0)
    assert np.all(np.abs(q[5].astype(int)) == 127)


@pytest.mark.parametrize("K,dtype", [(1024, "fp32"), (4096, "bf16")])
def test_pack_weights8_parity(qv, dev, K, dtype):
    W = synth.weights(384, K, seed=K + 1)
    if dtype == "bf16":
        W = synth.round_to_bf16(W)
    s = np.random.default_rng(2).uniform(0.5, 2.0, K).astype(np.float32)
    q, ws = run_quant8(qv, dev, W, dtype, s, weights=True)
    check_quant8(W, s, q, ws, f"int8 weights K={K} {dtype}")


def random_codes(rows, K, rng, lim=127):
    return rng.integers(-lim, lim + 1, size=(rows, K), dtype=np.int8)


def run_gemm8(qv, dev, Xq, xs, Wq, ws, bias=None, epi=0, out="fp32", ldy_pad=0):
    M, N = Xq.shape[0], Wq.shape[0]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ydt = torch.float32 if out == "fp32" else torch.bfloat16
    Yfull, Y = guarded_output(M, N, ydt, dev, ldy_pad)
    qv.qv_w8a8_gemm(t(Xq), t(xs), t(Wq), t(ws), None if bias is None else t(bias), Y, epi)
    torch.cuda.synchronize()
    check_guard(Yfull, M, N, f"w8a8 gemm M={M} N={N}")
    return Y.float().cpu().numpy()


@pytest.mark.parametrize("M,N,K,lim", [(1, 128, 64, 127), (37, 256, 1024, 127), (1374, 1024, 1024, 127),
                                       (130, 128, 4096, 63), (255, 384, 192, 127), (64, 128, 65536, 15)])
def test_gemm8_int32_accumulators_exact(qv, dev, M, N, K, lim):
    """Unit scales and fp32 output make Y the integer accumulator (|acc| < 2^24 by the code range)."""
    rng = np.random.default_rng(M * N + K)
    Xq, Wq = random_codes(M, K, rng, lim), random_codes(N, K, rng, lim)
    assert lim * lim * K < 2 ** 24
    Y = run_gemm8(qv, dev, Xq, np.ones(M, np.float32), Wq, np.ones(N, np.float32))
    np.testing.assert_array_equal(Y, oracle.gemm_int(Xq, Wq).astype(np.float32))


def test_gemm8_extreme_codes(qv, dev):
    M, N, K = 129, 256, 1024
    Xq = np.full((M, K), -128, np.int8)
    Wq = np.full((N, K), -128, np.int8)
    Y = run_gemm8(qv, dev, Xq, np.full(M, 2.0 ** -10, np.float32), Wq, np.full(N, 2.0 ** -10, np.float32))
    assert np.all(Y == 16384.0 * K * 2.0 ** -20)   # acc = 2^14 K = 2^24, exact


@pytest.mark.parametrize("epi,out,bias,pad", [(0, "fp32", False, 0), (1, "fp32", True, 0), (1, "bf16", False, 0),
                                              (0, "bf16", True, 64), (1, "bf16", True, 0), (0, "bf16", False, 8)])
def test_gemm8_epilogue_parity(qv, dev, epi, out, bias, pad):
    M, N, K = 1375, 384, 1024
    X = synth.vggt_activations(M, K, seed=15, dtype="bf16")
    W = synth.weights(N, K, seed=16)
    Xq, xs = oracle.hadamard_smooth_quant8(X, None, oracle.ROT_FWHT)
    Wq, ws = oracle.pack_weights8(W, None, oracle.ROT_FWHT)
    b = (0.1 * np.random.default_rng(1).standard_normal(N)).astype(np.float32) if bias else None
    Y = run_gemm8(qv, dev, Xq, xs, Wq, ws, b, epi, out, pad)
    acc.check_outputs(Y, oracle.w8a8_gemm(Xq, xs, Wq, ws, b, epi), out == "bf16", f"w8a8 epi={epi} out={out}")


def test_gemm8_many_tiles_per_block(qv, dev):
    M, N, K = 128 * 1700 + 77, 256, 256
    rng = np.random.default_rng(5)
    Xq, Wq = random_codes(M, K, rng), random_codes(N, K, rng)
    xs = rng.uniform(0.001, 0.01, M).astype(np.float32)
    ws = rng.uniform(0.001, 0.01, N).astype(np.float32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    Yfull, Y = guarded_output(M, N, torch.bfloat16, dev)
    qv.qv_w8a8_gemm(t(Xq), t(xs), t(Wq), t(ws), None, Y, 1)
    torch.cuda.synchronize()
    check_guard(Yfull, M, N, "w8a8 many tiles")
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 200, M), rng.choice(M, 300, replace=False)]))
    Yr = Y[torch.from_numpy(rows).to(dev)].float().cpu().numpy()
    acc.check_outputs(Yr, oracle.w8a8_gemm(Xq[rows], xs[rows], Wq, ws, None, 1), True, "w8a8 many tiles")
    assert not torch.isnan(Y.float()).any()


def test_w8a8_linear_end_to_end(qv, dev):
    """One frame, 1024 -> 1024, fp32 in and out, smoothing from frame 0: codes, scales and outputs
    against the oracle; the linear equals its two steps bitwise; W8A8 error below W4A4 error."""
    M, K, N = 1374, 1024, 1024
    X = synth.vggt_activations(M, K, seed=0)
    W = synth.weights(N, K, seed=1)
    s, inv = oracle.smoothing(oracle.rotate(X, oracle.ROT_FWHT), oracle.rotate(W, oracle.ROT_FWHT), 0.5)
    Wd = to_dev(W, "fp32", dev)
    Wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    ws = torch.empty((N,), device=dev)
    qv.qv_pack_weights8(Wd, torch.from_numpy(s).to(dev), Wq, ws)
    Xd = to_dev(X, "fp32", dev)
    invd = torch.from_numpy(inv).to(dev)
    Xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xs = torch.empty((M,), device=dev)
    qv.qv_hadamard_smooth_quant8(Xd, invd, Xq, xs)
    Y1 = torch.empty((M, N), device=dev)
    qv.qv_w8a8_gemm(Xq, xs, Wq, ws, None, Y1)
    work = torch.empty((qv.qv_w8a8_linear_workspace_size(M, K),), dtype=torch.uint8, device=dev)
    Y2 = torch.empty((M, N), device=dev)
    qv.qv_w8a8_linear(Xd, invd, Wq, ws, None, Y2, work)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    _, wc, ws_ref = check_quant8(W, s, Wq.cpu().numpy(), ws.cpu().numpy(), "w8 weights")
    _, xc, xs_ref = check_quant8(X, inv, Xq.cpu().numpy(), xs.cpu().numpy(), "w8 activations")
    Y = Y1.cpu().numpy()
    acc.check_outputs(Y, oracle.w8a8_gemm(xc, xs_ref, wc, ws_ref), False, "w8a8 linear")
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    e8 = np.linalg.norm(Y - ref) / np.linalg.norm(ref)
    Wq4, ws4 = oracle.pack_weights(W, s, oracle.ROT_FWHT)
    e4 = np.linalg.norm(oracle.w4a4_linear(X, inv, Wq4, ws4, mode=oracle.ROT_FWHT) - ref) / np.linalg.norm(ref)
    print(f"relative Frobenius error vs fp64 XW^T: W8A8 {e8:.5f}, W4A4 {e4:.5f}")
    assert e8 < e4 / 5
