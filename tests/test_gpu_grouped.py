"""Group-wise granularity on the GPU against the oracle.

Reading ([P4] "十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com), 双平滑细粒度量化（DSFQ） > 细粒度量化粒度,
truncated on the page): the pre-global rotation and the smoothing are unchanged; each row is then
quantized in groups of 128, 256 or 512 channels, each with its own absmax / 7 scale, and the
product sums the groups' integer dot products, each dequantized by its own pair of scales.

Codes and scales follow the per-token rules with the group's scale (tests/acceptance.py,
code_bounds_grouped); outputs allow, besides the relative bar, the fp32 accumulation over the groups
(check_outputs_grouped).  With unit scales the grouped product is an integer below 2^24 and must be
bit-exact.
"""
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


def t_(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_dev(a, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def smoothing_for(X, W):
    Xc = X[:min(len(X), synth.FRAME_TOKENS)]
    return oracle.smoothing(oracle.rotate(Xc, oracle.ROT_FWHT), oracle.rotate(W, oracle.ROT_FWHT), 0.5)


def quant_grouped(qv, dev, X, dtype, mult, group, weights=False):
    R, K = X.shape
    Xd = to_dev(X, dtype, dev)
    qfull, q, sfull, s = guarded_codes(R, K // 2, K // group, dev)
    s.fill_(float("nan"))
    m = None if mult is None else t_(mult.astype(np.float32), dev)
    if weights:
        qv.qv_pack_weights_grouped(Xd, m, group, q, s)
    else:
        qv.qv_hadamard_smooth_quant_grouped(Xd, m, group, q, s)
    torch.cuda.synchronize()
    check_codes_guard(qfull, sfull, R, label=f"grouped rotate-quantize R={R} K={K}")
    Xin = Xd.float().cpu().numpy().astype(np.float64)  # the values the kernel read (bf16-rounded)
    return q.cpu().numpy(), s.cpu().numpy(), Xin


def check_quant_grouped(q_gpu, s_gpu, Xin, mult, group, label):
    Xh = oracle.rotate(Xin, oracle.ROT_FWHT)
    q_ref, s_ref = oracle.quantize_groups(Xh, mult, group)
    t, tau, _, rel = acc.code_bounds_grouped(Xin, mult, group, Xh)
    qg = oracle.unpack_int4(q_gpu)
    rate = acc.check_codes(qg, q_ref, t, tau, label)
    assert not np.isnan(s_gpu).any(), f"{label}: a group scale was not written"
    acc.check_scales(s_gpu, s_ref, rel, label)
    return rate, np.where(qg != q_ref, qg, q_ref), s_ref


@pytest.mark.parametrize("K", [1024, 4096])
@pytest.mark.parametrize("group", [128, 256, 512])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_grouped_rotate_quant_parity(qv, dev, K, group, dtype):
    M = 1375 if K == 1024 else 333  # ragged: one row past a 4-row (K = 1024) wave group
    X = synth.vggt_activations(M, K, seed=K + group, dtype=dtype)
    W = synth.weights(256, K, seed=group)
    s, inv = smoothing_for(X, W)
    q, sc, Xin = quant_grouped(qv, dev, X, dtype, inv, group)
    rate, _, _ = check_quant_grouped(q, sc, Xin, inv, group, f"grouped K={K} g={group} {dtype}")
    print(f"grouped rotate-quantize K={K} group={group} {dtype}: mismatch {rate:.1e}")


@pytest.mark.parametrize("K,group", [(1024, 128), (4096, 512)])
def test_grouped_pack_weights_parity(qv, dev, K, group):
    N = 384
    W = synth.weights(N, K, seed=7)
    X = synth.vggt_activations(1374, K, seed=8, dtype="bf16")
    s, inv = smoothing_for(X, W)
    q, sc, Win = quant_grouped(qv, dev, W, "fp32", s, group, weights=True)
    check_quant_grouped(q, sc, Win, s, group, f"grouped weights K={K} g={group}")


def test_grouped_zero_group_and_zero_row(qv, dev):
    """A row whose rotated, smoothed values vanish on one group (x = t H / sqrt(K) with t zero
    there) gets scale 0 and zero codes in that group only; an all-zero row is zero throughout."""
    K, group = 1024, 128
    rng = np.random.default_rng(5)
    t = rng.integers(-13, 14, size=(6, K)).astype(np.float64) / 2.0
    t[1, 256:384] = 0.0
    t[4] = 0.0
    X = t @ oracle.hadamard(K).astype(np.float64) / np.sqrt(K)
    q, sc, Xin = quant_grouped(qv, dev, X, "fp32", None, group)
    assert sc[1, 2] == 0 and np.all(oracle.unpack_int4(q)[1, 256:384] == 0) and sc[1, 1] > 0
    assert np.all(sc[4] == 0) and np.all(q[4] == 0)
    check_quant_grouped(q, sc, Xin, None, group, "zero group")


def random_packed(rows, K, rng):
    return rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)


def run_gemm_grouped(qv, dev, Xq, xs, Wq, ws, group, bias=None, epi=0, out="fp32"):
    M, N = Xq.shape[0], Wq.shape[0]
    Yfull, Y = guarded_output(M, N, torch.float32 if out == "fp32" else torch.bfloat16, dev)
    qv.qv_w4a4_gemm_grouped(t_(Xq, dev), t_(xs, dev), t_(Wq, dev), t_(ws, dev), None if bias is None else t_(bias, dev),
                            Y, group, epi)
    torch.cuda.synchronize()
    check_guard(Yfull, M, N, f"grouped gemm M={M} N={N}")
    return Y.float().cpu().numpy()


@pytest.mark.parametrize("M,N,K,group", [(1, 128, 1024, 128), (200, 256, 1024, 256), (130, 128, 4096, 128),
                                         (77, 384, 4096, 512), (129, 128, 512, 128)])
def test_grouped_gemm_exact_with_unit_scales(qv, dev, M, N, K, group):
    """Unit scales: every group's contribution is its integer dot product, the sum stays below 2^24,
    so the fp32 output equals the oracle's integer product exactly."""
    rng = np.random.default_rng(M + K + group)
    Xq, Wq = random_packed(M, K, rng), random_packed(N, K, rng)
    ones_x = np.ones((M, K // group), np.float32)
    ones_w = np.ones((N, K // group), np.float32)
    Y = run_gemm_grouped(qv, dev, Xq, ones_x, Wq, ones_w, group)
    ref = oracle.gemm_int(oracle.unpack_int4(Xq), oracle.unpack_int4(Wq)).astype(np.float64)
    np.testing.assert_array_equal(Y, ref)


@pytest.mark.parametrize("group,epi,out,bias", [(128, 0, "fp32", False), (128, 1, "bf16", True), (256, 1, "fp32", False),
                                                (512, 0, "bf16", False), (128, 1, "fp32", True)])
def test_grouped_gemm_epilogue_parity(qv, dev, group, epi, out, bias):
    M, N, K = 1375, 384, 1024
    X = synth.vggt_activations(M, K, seed=15, dtype="bf16")
    W = synth.weights(N, K, seed=16)
    s, inv = smoothing_for(X, W)
    Xq, xs = oracle.hadamard_smooth_quant_grouped(X, inv, group, oracle.ROT_FWHT)
    Wq, ws = oracle.pack_weights_grouped(W, s, group, oracle.ROT_FWHT)
    b = (0.1 * np.random.default_rng(2).standard_normal(N)).astype(np.float32) if bias else None
    Y = run_gemm_grouped(qv, dev, Xq, xs, Wq, ws, group, b, epi, out)
    qa, qw = oracle.unpack_int4(Xq), oracle.unpack_int4(Wq)
    Y_ref = oracle.dequant_grouped(qa, qw, xs, ws, b, epi)
    worst = acc.check_outputs_grouped(Y, Y_ref, acc.grouped_abs_sum(qa, qw, xs, ws), out == "bf16", K // group,
                                      f"grouped g={group} epi={epi} {out} bias={bias}")
    print(f"grouped GEMM g={group} epi={epi} {out} bias={bias}: worst {worst:.2f} of the bound")


def test_grouped_gemm_many_tiles(qv, dev):
    """More tiles than resident blocks, ragged last row tile, bf16 + GELU; sampled rows checked."""
    M, N, K, group = 128 * 600 + 45, 256, 1024, 128
    rng = np.random.default_rng(17)
    Xq, Wq = random_packed(M, K, rng), random_packed(N, K, rng)
    xs = rng.uniform(0.001, 0.02, (M, K // group)).astype(np.float32)
    ws = rng.uniform(0.001, 0.02, (N, K // group)).astype(np.float32)
    Y = run_gemm_grouped(qv, dev, Xq, xs, Wq, ws, group, None, 1, "bf16")
    assert not np.isnan(Y).any(), "an output was not written"
    rows = np.unique(np.concatenate([np.arange(40), np.arange(M - 100, M), rng.choice(M, 200, replace=False)]))
    qa, qw = oracle.unpack_int4(Xq[rows]), oracle.unpack_int4(Wq)
    Y_ref = oracle.dequant_grouped(qa, qw, xs[rows], ws, None, 1)
    acc.check_outputs_grouped(Y[rows], Y_ref, acc.grouped_abs_sum(qa, qw, xs[rows], ws), True, K // group,
                              "grouped many tiles")


@pytest.mark.parametrize("K,group", [(1024, 128), (4096, 256)])
def test_grouped_linear_end_to_end(qv, dev, K, group):
    """qv_w4a4_linear_grouped equals its two steps bit for bit, and against the oracle the codes
    follow the grouped rules and the outputs (from the GPU's codes where they differ) the bound."""
    M, N = 1374, 256
    X = synth.vggt_activations(M, K, seed=20, dtype="bf16")
    W = synth.weights(N, K, seed=21)
    s, inv = smoothing_for(X, W)
    Xd, Wd = to_dev(X, "bf16", dev), to_dev(W, "fp32", dev)
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((N, K // group), dtype=torch.float32, device=dev)
    qv.qv_pack_weights_grouped(Wd, t_(s, dev), group, Wq, ws)
    Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, K // group), dtype=torch.float32, device=dev)
    invd = t_(inv, dev)
    qv.qv_hadamard_smooth_quant_grouped(Xd, invd, group, Xq, xs)
    Y1 = torch.empty((M, N), dtype=torch.float32, device=dev)
    qv.qv_w4a4_gemm_grouped(Xq, xs, Wq, ws, None, Y1, group, 1)
    work = torch.empty((qv.qv_w4a4_linear_grouped_workspace_size(M, K, group),), dtype=torch.uint8, device=dev)
    Y2 = torch.empty((M, N), dtype=torch.float32, device=dev)
    qv.qv_w4a4_linear_grouped(Xd, invd, group, Wq, ws, None, Y2, work, 1)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    Xin = Xd.float().cpu().numpy().astype(np.float64)
    _, qx, sx = check_quant_grouped(Xq.cpu().numpy(), xs.cpu().numpy(), Xin, inv, group, "linear activations")
    _, qw, sw = check_quant_grouped(Wq.cpu().numpy(), ws.cpu().numpy(), W.astype(np.float64), s, group,
                                    "linear weights")
    # outputs from the GPU's codes and scales (differences in codes are checked above)
    qa_g, qw_g = oracle.unpack_int4(Xq.cpu().numpy()), oracle.unpack_int4(Wq.cpu().numpy())
    xs_g, ws_g = xs.cpu().numpy(), ws.cpu().numpy()
    Y_ref = oracle.dequant_grouped(qa_g, qw_g, xs_g, ws_g, None, 1)
    acc.check_outputs_grouped(Y1.cpu().numpy(), Y_ref, acc.grouped_abs_sum(qa_g, qw_g, xs_g, ws_g), False, K // group,
                              "grouped linear")
