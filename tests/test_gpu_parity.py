"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded VGGT-shaped inputs.

Rules (tests/acceptance.py): int32 accumulators bit-exact on identical codes; int4 codes
admissible everywhere and mismatched at <= 1e-4 (only at fp32 near-ties); outputs within 1e-3
relative error (fp32) or one bf16 ulp (bf16) of the oracle's dequantization of the GPU's codes.
Sources: page "十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com), 训练后量化（PTQ） and
双平滑细粒度量化（DSFQ）.
"""
import math

import numpy as np
import pytest

import acceptance as acc
from guard import check_codes_guard, check_guard, guarded_codes, guarded_output
import oracle
from bit_ptq_reconstruction_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


def smoothing_for(X, W, mode=oracle.ROT_EXPLICIT):
    """Smoothing factors from frame 0 of the activations (at most 1374 rows) and the weights."""
    Xc = X[:min(len(X), synth.FRAME_TOKENS)]
    return oracle.smoothing(oracle.rotate(Xc, mode), oracle.rotate(W, mode), 0.5)


def run_quant(qv, dev, X, dtype, mult, ld_pad=0, weights=False):
    M, K = X.shape
    Xd = to_dev(np.pad(X, ((0, 0), (0, ld_pad))) if ld_pad else X, dtype, dev)
    if ld_pad:
        Xd = Xd[:, :K]
    md = None if mult is None else torch.from_numpy(mult).to(dev)
    qfull, q, sfull, s = guarded_codes(M, K // 2, 0, dev)
    (qv.qv_pack_weights if weights else qv.qv_hadamard_smooth_quant)(Xd, md, q, s)
    torch.cuda.synchronize()
    check_codes_guard(qfull, sfull, M, label=f"rotate-quantize M={M} K={K}")
    return q.cpu().numpy(), s.cpu().numpy()


def check_quant_against_oracle(X, mult, q_packed, s_gpu, mode, label):
    Xhat = oracle.rotate(X, mode)
    q_ref, s_ref = oracle.quantize_rows(Xhat, mult)
    t, tau, _, rel_scale = acc.code_bounds(X, mult, Xhat)
    q_gpu = oracle.unpack_int4(q_packed)
    rate = acc.check_codes(q_gpu, q_ref, t, tau, label)
    acc.check_scales(s_gpu, s_ref, rel_scale, label)
    # The oracle's codes, with the GPU's admissible near-tie codes where the two differ.
    return rate, np.where(q_gpu != q_ref, q_gpu, q_ref), s_ref


# ---------------------------------------------------------------------------- rotate-quantize

@pytest.mark.parametrize("K,dtype,M,smooth,pad", [
    (1024, "fp32", 1, True, 0), (1024, "fp32", 5, False, 0), (1024, "bf16", 1374, True, 0),
    (1024, "fp32", 1375, True, 64), (4096, "bf16", 1, True, 0), (4096, "bf16", 137, True, 0),
    (4096, "fp32", 70, False, 32), (1024, "bf16", 257, True, 8),
    # bf16 rows take the matrix-core kernel: padded rows, an odd row count (the last group of a
    # 2-row wave is half empty at width 1024), and enough rows that every wave transforms several
    # groups with the next group's loads in flight
    (4096, "bf16", 7001, True, 8), (1024, "bf16", 20001, True, 8), (1024, "bf16", 1, False, 0),
])
def test_hadamard_smooth_quant_parity(qv, dev, K, dtype, M, smooth, pad):
    X = synth.vggt_activations(M, K, seed=K + M, dtype=dtype)
    W = synth.weights(128, K, seed=3)
    mult = smoothing_for(X, W)[1] if smooth else None
    q, s = run_quant(qv, dev, X, dtype, mult, ld_pad=pad)
    rate, _, _ = check_quant_against_oracle(X, mult, q, s, oracle.ROT_EXPLICIT, f"K={K} {dtype} M={M}")
    print(f"K={K} {dtype} M={M}: code mismatch rate {rate:.2e}")


@pytest.mark.parametrize("K,dtype", [(1024, "fp32"), (1024, "bf16"), (4096, "bf16"), (4096, "fp32")])
def test_pack_weights_parity(qv, dev, K, dtype):
    N = 384
    X = synth.vggt_activations(300, K, seed=7, dtype=dtype)
    W = synth.weights(N, K, seed=8)
    if dtype == "bf16":
        W = synth.round_to_bf16(W)
    s, _ = smoothing_for(X, W)
    q, ws = run_quant(qv, dev, W, dtype, s, weights=True)
    check_quant_against_oracle(W, s, q, ws, oracle.ROT_EXPLICIT, f"weights K={K} {dtype}")


@pytest.mark.parametrize("K", [1024, 4096])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_constructed_ties_are_bit_exact(qv, dev, K, dtype):
    """Code-space targets on half-integers: the rotated row is exactly t, the scale exactly 1, so
    every code is round-half-even(t) with no tolerance (tests/golden/quant_ties.txt)."""
    import scipy.linalg

    t = np.array([float(r.split()[0]) for r in open(__file__.replace("test_gpu_parity.py", "golden/quant_ties.txt"))
                  if r.strip() and not r.startswith("#")])
    rng = np.random.default_rng(K)
    rows = []
    for i in range(9):
        target = np.zeros(K)
        pos = rng.choice(K, size=len(t), replace=False) if i else np.arange(len(t))
        target[pos] = rng.permutation(t) if i else t
        rows.append(target)
    T = np.array(rows)
    H = scipy.linalg.hadamard(K).astype(np.float64)
    X = (T @ H) / math.sqrt(K)
    assert np.all(X.astype(np.float32) == X) and (dtype == "fp32" or np.all(synth.round_to_bf16(X) == X))
    q, s = run_quant(qv, dev, X.astype(np.float32), dtype, None)
    np.testing.assert_array_equal(s, np.ones(len(rows), np.float32))
    np.testing.assert_array_equal(oracle.unpack_int4(q), np.rint(T).astype(np.int8))


@pytest.mark.parametrize("K", [1024, 4096])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])  # bf16 rows take the matrix-core kernel
def test_zero_tiny_and_outlier_rows(qv, dev, K, dtype):
    X = np.zeros((6, K), np.float32)
    X[1, :] = 1e-41 if dtype == "fp32" else 1e-39  # subnormal row: subnormal scale -> all-zero row
    X[2, 17] = 1000.0          # one-hot outlier: spreads flat, every code +-7
    X[3, :] = 2.5              # constant row: a single spike
    X[4] = synth.vggt_activations(1, K, seed=1, dtype=dtype)[0]
    X[5, ::2] = -3.0
    if dtype == "bf16":
        X = synth.round_to_bf16(X)
        assert X[1, 0] != 0 and abs(X[1, 0]) < 2.0 ** -126  # still a (bf16) subnormal
    q, s = run_quant(qv, dev, X, dtype, None)
    assert s[0] == 0 and s[1] == 0
    codes = oracle.unpack_int4(q)
    assert np.all(codes[0] == 0) and np.all(codes[1] == 0)
    assert np.all(np.abs(codes[2]) == 7)
    assert codes[3, 0] == 7 and np.all(codes[3, 1:] == 0)
    check_quant_against_oracle(X, None, q, s, oracle.ROT_EXPLICIT, f"special rows K={K} {dtype}")


@pytest.mark.parametrize("K", [1024, 4096])
def test_cancellation_rows(qv, dev, K):
    """bf16 rows built so that the 32-element groups the matrix-core kernel contracts first cancel:
    x_k = big * (-1)^popcount(k & pattern) (1 + 2^-7 noise) + unit noise.  One output of each
    32-point transform gathers the groups constructively; the other 31 are what is left of 32 large
    terms of opposite signs, which is where fp32 summation order matters most."""
    rng = np.random.default_rng(K + 11)
    M = 48
    k = np.arange(K)
    X = np.empty((M, K), np.float32)
    for m in range(M):
        big = 10.0 ** rng.uniform(0, 4)
        pattern = int(rng.integers(0, 32))
        sign = np.where(np.array([bin(int(v) & pattern).count("1") % 2 for v in k]), -1.0, 1.0)
        X[m] = big * sign * (1 + rng.standard_normal(K) * 2.0 ** -7) + rng.standard_normal(K)
    X = synth.round_to_bf16(X)
    q, s = run_quant(qv, dev, X, "bf16", None)
    rate, _, _ = check_quant_against_oracle(X, None, q, s, oracle.ROT_EXPLICIT, f"cancellation rows K={K}")
    print(f"cancellation rows K={K}: code mismatch rate {rate:.2e}")


# ---------------------------------------------------------------------------- int4 GEMM

def random_packed(rows, K, rng, fill=None):
    if fill is None:
        return rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    code = fill & 0xF
    return np.full((rows, K // 2), code | (code << 4), dtype=np.uint8)


def run_gemm(qv, dev, Xq, xs, Wq, ws, bias=None, epi=0, out="fp32", ldy_pad=0):
    M, N = Xq.shape[0], Wq.shape[0]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ydt = torch.float32 if out == "fp32" else torch.bfloat16
    Yfull, Y = guarded_output(M, N, ydt, dev, ldy_pad)
    qv.qv_w4a4_gemm(t(Xq), t(xs), t(Wq), t(ws), None if bias is None else t(bias), Y, epi)
    torch.cuda.synchronize()
    check_guard(Yfull, M, N, f"gemm M={M} N={N}")
    return Y.float().cpu().numpy()


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (37, 256, 1024), (1374, 1024, 1024), (130, 128, 4096),
                                   (255, 384, 2048), (64, 128, 65536)])
def test_gemm_int32_accumulators_exact(qv, dev, M, N, K):
    """Scales of 1 and an fp32 output make Y the integer accumulator itself (|acc| < 2^24)."""
    rng = np.random.default_rng(M * N + K)
    Xq, Wq = random_packed(M, K, rng), random_packed(N, K, rng)
    Y = run_gemm(qv, dev, Xq, np.ones(M, np.float32), Wq, np.ones(N, np.float32))
    _, accum = oracle.w4a4_gemm(Xq, np.ones(M, np.float32), Wq, np.ones(N, np.float32), return_acc=True)
    np.testing.assert_array_equal(Y, accum.astype(np.float32))


@pytest.mark.parametrize("fa,fw", [(-8, -8), (7, 7), (7, -8), (-1, 1)])
def test_gemm_extreme_codes(qv, dev, fa, fw):
    rng = np.random.default_rng(0)
    M, N, K = 129, 256, 65536
    Xq, Wq = random_packed(M, K, rng, fa), random_packed(N, K, rng, fw)
    Y = run_gemm(qv, dev, Xq, np.ones(M, np.float32), Wq, np.ones(N, np.float32))
    assert np.all(Y == fa * fw * K)


def test_gemm_tiny_row_scales(qv, dev):
    """Row scales just above the fp32 normal minimum (the epilogue folds 2^-8 into them, which makes
    them subnormal there) still give outputs within the relative bound."""
    M, N, K = 130, 256, 1024
    rng = np.random.default_rng(11)
    Xq, Wq = random_packed(M, K, rng), random_packed(N, K, rng)
    xs = (rng.uniform(1.0, 2.0, M) * 2.0 ** rng.integers(-126, -116, M)).astype(np.float32)
    xs[:4] = [2.0 ** -126, 1.2345 * 2.0 ** -124, 1.999 * 2.0 ** -119, 3.0]
    ws = rng.uniform(0.001, 0.02, N).astype(np.float32)
    for epi in (0, 1):
        Y = run_gemm(qv, dev, Xq, xs, Wq, ws, None, epi, "fp32")
        Y_ref = oracle.w4a4_gemm(Xq, xs, Wq, ws, None, epi)
        acc.check_outputs(Y, Y_ref, False, f"tiny row scales epi={epi}")


@pytest.mark.parametrize("out", ["fp32", "bf16"])
def test_gelu_epilogue_sweep(qv, dev, out):
    """The GELU epilogue over y in [-13.9, 10.4], out to the tail where fp32 outputs turn subnormal:
    every accumulator is 1 (one code pair of 1 at k = 0), so y = x_scale[m] w_scale[n] spans a dense
    grid.  fp32 outputs (degree-5 fit) must stay within 1e-4 relative, bf16 outputs within 1 ulp."""
    M, N, K = 4096, 256, 128
    Xq = np.zeros((M, K // 2), dtype=np.uint8)
    Wq = np.zeros((N, K // 2), dtype=np.uint8)
    Xq[:, 0] = 1
    Wq[:, 0] = 1
    xs = np.linspace(-13.4, 10.0, M).astype(np.float32)
    ws = (1.0 + np.arange(N) * (0.04 / N)).astype(np.float32)
    Y = run_gemm(qv, dev, Xq, xs, Wq, ws, None, 1, out)
    Y_ref = oracle.w4a4_gemm(Xq, xs, Wq, ws, None, 1)
    worst = acc.check_outputs(Y, Y_ref, out == "bf16", f"GELU sweep ({out})")
    if out == "fp32":
        assert worst <= 1e-4, f"GELU sweep: max relative error {worst:.2e}"
    print(f"GELU sweep {out}: worst {worst:.2e} ({'bf16 ulps' if out == 'bf16' else 'relative'})")


@pytest.mark.parametrize("K,epi,bias", [(256, 0, False), (256, 1, True), (1024, 0, False)])
def test_gemm_many_tiles_per_block(qv, dev, K, epi, bias):
    """bf16 outputs over more tiles than resident blocks (each block walks several tiles, its LDS ring
    streaming across tile boundaries), down to two stages per tile, with a ragged last row tile;
    every output of a sample of rows is checked."""
    M, N = 128 * 1700 + 77, 256
    rng = np.random.default_rng(K + epi)
    Xq, Wq = random_packed(M, K, rng), random_packed(N, K, rng)
    xs = rng.uniform(0.01, 0.1, M).astype(np.float32)
    ws = rng.uniform(0.01, 0.1, N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32) if bias else None
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    Yfull, Y = guarded_output(M, N, torch.bfloat16, dev)
    qv.qv_w4a4_gemm(t(Xq), t(xs), t(Wq), t(ws), None if b is None else t(b), Y, epi)
    torch.cuda.synchronize()
    check_guard(Yfull, M, N, "many tiles")
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 200, M), rng.choice(M, 300, replace=False)]))
    Yr = Y[torch.from_numpy(rows).to(dev)].float().cpu().numpy()
    Y_ref = oracle.w4a4_gemm(Xq[rows], xs[rows], Wq, ws, b, epi)
    acc.check_outputs(Yr, Y_ref, True, f"many tiles K={K} epi={epi} bias={bias}")
    assert not torch.isnan(Y.float()).any(), "an output element was not written"


@pytest.mark.parametrize("epi,out,bias,pad", [(0, "fp32", False, 0), (1, "fp32", False, 0), (0, "bf16", False, 0),
                                              (1, "bf16", True, 64), (0, "fp32", True, 32), (0, "bf16", True, 0),
                                              (1, "bf16", False, 8)])
def test_gemm_epilogue_parity(qv, dev, epi, out, bias, pad):
    """Every epilogue instance (GELU or not, bias or not, fp32 or bf16 outputs) on a ragged row count
    (1375 rows: a partial last tile for every tile height) against the oracle."""
    M, N, K = 1375, 384, 1024
    X = synth.vggt_activations(M, K, seed=5, dtype="bf16")
    W = synth.weights(N, K, seed=6)
    s, inv = smoothing_for(X, W)
    Xq, xs = oracle.hadamard_smooth_quant(X, inv, oracle.ROT_FWHT)
    Wq, ws = oracle.pack_weights(W, s, oracle.ROT_FWHT)
    b = (0.1 * np.random.default_rng(1).standard_normal(N)).astype(np.float32) if bias else None
    Y = run_gemm(qv, dev, Xq, xs, Wq, ws, b, epi, out, pad)
    Y_ref = oracle.w4a4_gemm(Xq, xs, Wq, ws, b, epi)
    worst = acc.check_outputs(Y, Y_ref, out == "bf16", f"epi={epi} out={out} bias={bias}")
    print(f"epilogue epi={epi} out={out} bias={bias}: max rel err {worst:.2e}")


@pytest.mark.parametrize("K,dtype", [(1024, "bf16"), (4096, "bf16"), (1024, "fp32")])
def test_row_ranges_are_independent(qv, dev, K, dtype):
    """Rows are independent through both online steps: calls on row ranges give bit-identical codes,
    scales and outputs to one call over all rows.  The split offsets are multiples of 4 rows (the
    scale vectors' 16-byte alignment) and of no tile height, so a caller may split M into chunks."""
    M, N = 3000, 384
    X = synth.vggt_activations(M, K, seed=21, dtype=dtype)
    W = synth.weights(N, K, seed=22)
    Xd, Wd = to_dev(X, dtype, dev), to_dev(W, "fp32", dev)
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((N,), dtype=torch.float32, device=dev)
    qv.qv_pack_weights(Wd, None, Wq, ws)
    whole = [torch.empty((M, K // 2), dtype=torch.uint8, device=dev), torch.empty((M,), dtype=torch.float32, device=dev),
             torch.empty((M, N), dtype=torch.bfloat16, device=dev)]
    parts = [torch.empty_like(t) for t in whole]
    qv.qv_hadamard_smooth_quant(Xd, None, whole[0], whole[1])
    qv.qv_w4a4_gemm(whole[0], whole[1], Wq, ws, None, whole[2], 1)
    for a, b in ((0, 4), (4, 1004), (1004, 2996), (2996, 3000)):
        qv.qv_hadamard_smooth_quant(Xd[a:b], None, parts[0][a:b], parts[1][a:b])
        qv.qv_w4a4_gemm(parts[0][a:b], parts[1][a:b], Wq, ws, None, parts[2][a:b], 1)
    torch.cuda.synchronize()
    for w, p_ in zip(whole, parts):
        assert torch.equal(w.view(torch.uint8), p_.view(torch.uint8))


def test_concurrent_streams_match_one_stream(qv, dev):
    """Two linears issued on two streams at once (each call on its caller's stream, kernels of both
    in flight together) give the bit-identical codes, scales and outputs of the same calls issued
    one after the other on one stream: the library keeps no per-call state outside its arguments."""
    shapes = [(2000, 1024, 768, 1), (1500, 4096, 256, 0)]
    inputs = []
    for i, (M, K, N, epi) in enumerate(shapes):
        X = to_dev(synth.vggt_activations(M, K, seed=30 + i, dtype="bf16"), "bf16", dev)
        Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        ws = torch.empty((N,), dtype=torch.float32, device=dev)
        qv.qv_pack_weights(to_dev(synth.weights(N, K, seed=40 + i), "fp32", dev), None, Wq, ws)
        inputs.append((X, Wq, ws, epi))

    def outputs():
        return [(torch.empty((X.shape[0], X.shape[1] // 2), dtype=torch.uint8, device=dev),
                 torch.empty((X.shape[0],), dtype=torch.float32, device=dev),
                 torch.empty((X.shape[0], Wq.shape[0]), dtype=torch.bfloat16, device=dev)) for X, Wq, _, _ in inputs]

    def run(i, o, stream):
        X, Wq, ws, epi = inputs[i]
        qv.qv_hadamard_smooth_quant(X, None, o[0], o[1], stream)
        qv.qv_w4a4_gemm(o[0], o[1], Wq, ws, None, o[2], epi, stream)

    torch.cuda.synchronize()
    one = outputs()
    for rep in range(3):
        for i in range(len(inputs)):
            run(i, one[i], torch.cuda.current_stream())
    torch.cuda.synchronize()
    two = outputs()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for i in range(len(inputs)):
            run(i, two[i], streams[i])
    torch.cuda.synchronize()
    for a, b in zip(one, two):
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


# ---------------------------------------------------------------------------- whole layer

@pytest.mark.parametrize("K", [1024, 4096])
def test_linear_equals_its_two_steps_and_is_deterministic(qv, dev, K):
    M, N = 2000, 256
    X = synth.vggt_activations(M, K, seed=9, dtype="bf16")
    W = synth.weights(N, K, seed=10)
    Xd, Wd = to_dev(X, "bf16", dev), to_dev(W, "fp32", dev)
    sm = torch.ones(K, device=dev)
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((N,), dtype=torch.float32, device=dev)
    qv.qv_pack_weights(Wd, sm, Wq, ws)
    Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty((M,), dtype=torch.float32, device=dev)
    qv.qv_hadamard_smooth_quant(Xd, sm, Xq, xs)
    Y1 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qv.qv_w4a4_gemm(Xq, xs, Wq, ws, None, Y1, qv.QV_EPI_GELU)
    work = torch.empty((qv.qv_w4a4_linear_workspace_size(M, K),), dtype=torch.uint8, device=dev)
    outs = []
    for _ in range(3):
        Y2 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        qv.qv_w4a4_linear(Xd, sm, Wq, ws, None, Y2, work, qv.QV_EPI_GELU)
        outs.append(Y2)
    torch.cuda.synchronize()
    for Y2 in outs:
        assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))


def test_calls_run_on_the_given_stream(qv, dev):
    """Every call is ordered on the stream it is given: the whole layer issued on a side stream
    (default priority), after that stream waited for the inputs, equals the default-stream result."""
    M, K, N = 1500, 1024, 384
    X = synth.vggt_activations(M, K, seed=12, dtype="bf16")
    W = synth.weights(N, K, seed=13)
    Xd, Wd = to_dev(X, "bf16", dev), to_dev(W, "fp32", dev)
    sm = torch.ones(K, device=dev)
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((N,), dtype=torch.float32, device=dev)
    qv.qv_pack_weights(Wd, sm, Wq, ws)
    work = torch.empty((qv.qv_w4a4_linear_workspace_size(M, K),), dtype=torch.uint8, device=dev)
    Y1 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qv.qv_w4a4_linear(Xd, sm, Wq, ws, None, Y1, work, qv.QV_EPI_GELU)
    torch.cuda.synchronize()
    work2 = torch.empty_like(work)
    Y2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())  # the inputs and Y2's fill are complete first
    with torch.cuda.stream(side):
        qv.qv_w4a4_linear(Xd, sm, Wq, ws, None, Y2, work2, qv.QV_EPI_GELU)
        Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        xs = torch.empty((M,), dtype=torch.float32, device=dev)
        Y3 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
        qv.qv_hadamard_smooth_quant(Xd, sm, Xq, xs, stream=side)
        qv.qv_w4a4_gemm(Xq, xs, Wq, ws, None, Y3, qv.QV_EPI_GELU, stream=side)
    side.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(Y1.view(torch.int16), Y3.view(torch.int16))


def test_calls_replay_from_a_hip_graph(qv, dev):
    """The online calls record into a HIP graph (they launch kernels only: no memset, copy,
    allocation or synchronisation). A two-layer chain (1024 -> 4096 with GELU, then the 4096-wide
    rotation of that output -> 256) is captured once and replayed three times, with the outputs
    overwritten and eager work between replays; every replay equals the eager result bit for bit."""
    M, K1, N1, N2 = 2000, 1024, 4096, 256
    X = to_dev(synth.vggt_activations(M, K1, seed=21, dtype="bf16"), "bf16", dev)
    sm1, sm2 = torch.rand(K1, device=dev) + 0.5, torch.rand(N1, device=dev) + 0.5
    Wq1 = torch.empty((N1, K1 // 2), dtype=torch.uint8, device=dev)
    ws1 = torch.empty((N1,), dtype=torch.float32, device=dev)
    Wq2 = torch.empty((N2, N1 // 2), dtype=torch.uint8, device=dev)
    ws2 = torch.empty((N2,), dtype=torch.float32, device=dev)
    qv.qv_pack_weights(to_dev(synth.weights(N1, K1, seed=22), "fp32", dev), sm1, Wq1, ws1)
    qv.qv_pack_weights(to_dev(synth.weights(N2, N1, seed=23), "fp32", dev), sm2, Wq2, ws2)
    Xq = torch.empty((M, K1 // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty((M,), dtype=torch.float32, device=dev)
    Y1 = torch.empty((M, N1), dtype=torch.bfloat16, device=dev)
    Y2 = torch.empty((M, N2), dtype=torch.float32, device=dev)
    work = torch.empty((qv.qv_w4a4_linear_workspace_size(M, N1),), dtype=torch.uint8, device=dev)

    def chain():
        qv.qv_hadamard_smooth_quant(X, 1.0 / sm1, Xq, xs)
        qv.qv_w4a4_gemm(Xq, xs, Wq1, ws1, None, Y1, qv.QV_EPI_GELU)
        qv.qv_w4a4_linear(Y1, 1.0 / sm2, Wq2, ws2, None, Y2, work, qv.QV_EPI_NONE)

    inv1, inv2 = 1.0 / sm1, 1.0 / sm2

    def chain_fixed():  # the graph keeps the multipliers' addresses: no tensors made inside it
        qv.qv_hadamard_smooth_quant(X, inv1, Xq, xs)
        qv.qv_w4a4_gemm(Xq, xs, Wq1, ws1, None, Y1, qv.QV_EPI_GELU)
        qv.qv_w4a4_linear(Y1, inv2, Wq2, ws2, None, Y2, work, qv.QV_EPI_NONE)

    chain_fixed()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (Xq, xs, Y1, Y2)]
    assert torch.isfinite(ref[3]).all()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain_fixed()
    torch.cuda.synchronize()
    for r in range(3):
        chain()  # eager work between replays (same results, fresh multiplier tensors)
        Xq.fill_(0x55)
        xs.fill_(-1.0)
        Y1.fill_(float("nan"))
        Y2.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((Xq, xs, Y1, Y2), ref):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {r}"


def test_calls_from_several_host_threads(qv, dev):
    """Four host threads issue the layer concurrently, each on its own stream (default priority)
    with its own workspace and output; every result equals the single-threaded one bit for bit.
    The library's only host state is its per-device launch caches, which are atomics."""
    from concurrent.futures import ThreadPoolExecutor

    M, K, N = 1500, 4096, 256
    X = to_dev(synth.vggt_activations(M, K, seed=31, dtype="bf16"), "bf16", dev)
    inv = 1.0 / (torch.rand(K, device=dev) + 0.5)
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((N,), dtype=torch.float32, device=dev)
    qv.qv_pack_weights(to_dev(synth.weights(N, K, seed=32), "fp32", dev), 1.0 / inv, Wq, ws)
    nbytes = qv.qv_w4a4_linear_workspace_size(M, K)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qv.qv_w4a4_linear(X, inv, Wq, ws, None, ref, torch.empty((nbytes,), dtype=torch.uint8, device=dev),
                      qv.QV_EPI_GELU)
    torch.cuda.synchronize()
    jobs = []
    for _ in range(4):
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
        work = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
        stream = torch.cuda.Stream(device=dev)
        stream.wait_stream(torch.cuda.current_stream())  # inputs and the NaN fill are complete first
        jobs.append((Y, work, stream))

    def run(job):
        Y, work, stream = job
        for _ in range(10):
            qv.qv_w4a4_linear(X, inv, Wq, ws, None, Y, work, qv.QV_EPI_GELU, stream=stream)
        stream.synchronize()

    with ThreadPoolExecutor(len(jobs)) as pool:
        list(pool.map(run, jobs))
    for Y, _, _ in jobs:
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16))


def test_linear_against_oracle_end_to_end(qv, dev):
    """Single 1024->1024 linear on one frame (M = 1374), fp32 in and out, smoothing from frame 0."""
    M, K, N = 1374, 1024, 1024
    X = synth.vggt_activations(M, K, seed=0)
    W = synth.weights(N, K, seed=1)
    s, inv = smoothing_for(X, W)
    Wd = to_dev(W, "fp32", dev)
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((N,), dtype=torch.float32, device=dev)
    qv.qv_pack_weights(Wd, torch.from_numpy(s).to(dev), Wq, ws)
    Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty((M,), dtype=torch.float32, device=dev)
    qv.qv_hadamard_smooth_quant(to_dev(X, "fp32", dev), torch.from_numpy(inv).to(dev), Xq, xs)
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    qv.qv_w4a4_gemm(Xq, xs, Wq, ws, None, Y)
    torch.cuda.synchronize()
    _, wc, ws_ref = check_quant_against_oracle(W, s, Wq.cpu().numpy(), ws.cpu().numpy(), oracle.ROT_EXPLICIT,
                                               "weights")
    _, xc, xs_ref = check_quant_against_oracle(X, inv, Xq.cpu().numpy(), xs.cpu().numpy(), oracle.ROT_EXPLICIT,
                                               "activations")
    Y_ref = oracle.w4a4_gemm(oracle.pack_int4(xc), xs_ref, oracle.pack_int4(wc), ws_ref)
    acc.check_outputs(Y.cpu().numpy(), Y_ref, False, "linear")
    # Quantization quality (reported): relative Frobenius error against the fp64 product, next to
    # the oracle's own W4A4 error on the same inputs (the two must agree closely).
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    err = np.linalg.norm(Y.cpu().numpy() - ref) / np.linalg.norm(ref)
    Wq_o, ws_o = oracle.pack_weights(W, s)
    err_o = np.linalg.norm(oracle.w4a4_linear(X, inv, Wq_o, ws_o) - ref) / np.linalg.norm(ref)
    print(f"W4A4 relative Frobenius error vs fp64 XW^T: GPU {err:.5f}, oracle {err_o:.5f}")
    assert abs(err - err_o) <= 1e-3 * err_o


def test_zero_rows_give_bias_only(qv, dev):
    M, K, N = 4, 1024, 128
    X = np.zeros((M, K), np.float32)
    W = synth.weights(N, K, seed=2)
    bias = np.linspace(-1, 1, N).astype(np.float32)
    Wq, ws = oracle.pack_weights(W)
    Xq, xs = oracle.hadamard_smooth_quant(X)
    Y = run_gemm(qv, dev, Xq, xs, Wq, ws, bias)
    np.testing.assert_array_equal(Y, np.tile(bias, (M, 1)))


def test_empty_inputs_are_noops(qv, dev):
    K, N = 1024, 128
    X = torch.empty((0, K), device=dev)
    q = torch.empty((0, K // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((0,), device=dev)
    qv.qv_hadamard_smooth_quant(X, None, q, s)
    Wq = torch.zeros((N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.ones((N,), device=dev)
    Y = torch.empty((0, N), device=dev)
    qv.qv_w4a4_gemm(q, s, Wq, ws, None, Y)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------- calibration

@pytest.mark.parametrize("K,dtype", [(1024, "bf16"), (4096, "fp32")])
def test_smooth_calibrate_parity(qv, dev, K, dtype):
    X = synth.vggt_activations(1374, K, seed=4, dtype=dtype)
    W = synth.weights(512, K, seed=5)
    s_ref, inv_ref = smoothing_for(X, W, oracle.ROT_FWHT)
    s = torch.empty(K, device=dev)
    inv = torch.empty(K, device=dev)
    qv.qv_smooth_calibrate(to_dev(X, dtype, dev), to_dev(W, "fp32", dev), s, inv, 0.5)
    torch.cuda.synchronize()
    # The column maxima carry the butterfly rounding of one element (relative <= log2(K) u sum|x| /
    # (sqrt(K) max)), plus the fp32 pow/divide; 1e-4 relative covers both with margin on these rows.
    np.testing.assert_allclose(s.cpu().numpy(), s_ref, rtol=1e-4)
    np.testing.assert_allclose(inv.cpu().numpy(), inv_ref, rtol=1e-4)
