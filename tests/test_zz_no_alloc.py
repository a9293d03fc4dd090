"""The allocation-free linear (qv_w4a4_linear_noalloc) through the C ABI on the GPU: its output equals
that of qv_w4a4_linear with a caller workspace, on two calls in a row, the second with a smaller
input (the static scratch array keeps the first call's codes and scales, and the second call must
rewrite what it reads), and both against the oracle's dequantization of the codes.

Method: page "十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com), 训练后量化（PTQ） and 双平滑细粒度量化（DSFQ）:
rotate, smooth, quantize per token, integer GEMM, dequantize."""
import numpy as np
import pytest

import acceptance as acc
from guard import check_guard, guarded_output
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


def layer(qv, dev, M, K, N, seed):
    """Seeded bf16 activations, smoothing from frame 0, weights packed on the GPU."""
    X = synth.vggt_activations(M, K, seed=seed, dtype="bf16")
    W = synth.weights(N, K, seed=seed + 1)
    s, inv = oracle.smoothing(oracle.rotate(X[:min(M, synth.FRAME_TOKENS)], oracle.ROT_FWHT),
                              oracle.rotate(W, oracle.ROT_FWHT), 0.5)
    Xd = torch.from_numpy(X).to(dev).to(torch.bfloat16)
    Wd = torch.from_numpy(W).to(dev)
    sd, invd = torch.from_numpy(s).to(dev), torch.from_numpy(inv).to(dev)
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((N,), dtype=torch.float32, device=dev)
    qv.qv_pack_weights(Wd, sd, Wq, ws)
    return Xd, invd, Wq, ws


def test_noalloc_linear_equals_linear_on_two_calls(qv, dev):
    # first call: 9000 rows of width 1024 (about 4.6 MB of the 32 MiB array), with GELU;
    # second call: a smaller input, 1375 rows of width 4096 (2.8 MB), no epilogue.
    cases = [(9000, 1024, 1024, qv.QV_EPI_GELU, 7), (1375, 4096, 256, qv.QV_EPI_NONE, 11)]
    prepared = [layer(qv, dev, M, K, N, seed) for M, K, N, _, seed in cases]
    outs = []
    for (M, K, N, epi, _), (Xd, invd, Wq, ws) in zip(cases, prepared):
        print(f"noalloc call M={M} K={K} N={N} epi={epi}", flush=True)
        full, Y = guarded_output(M, N, torch.bfloat16, dev)
        qv.qv_w4a4_linear_noalloc(Xd, invd, Wq, ws, None, Y, epi)
        torch.cuda.synchronize()
        check_guard(full, M, N, f"noalloc M={M}")
        outs.append(Y.clone())
    for (M, K, N, epi, _), (Xd, invd, Wq, ws), Yn in zip(cases, prepared, outs):
        work = torch.empty((qv.qv_w4a4_linear_workspace_size(M, K),), dtype=torch.uint8, device=dev)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        qv.qv_w4a4_linear(Xd, invd, Wq, ws, None, Y, work, epi)
        torch.cuda.synchronize()
        assert torch.equal(Yn.view(torch.int16), Y.view(torch.int16)), f"M={M} K={K}: differs from qv_w4a4_linear"
        # and the same rows against the oracle (the workspace holds the codes and scales the call used)
        xq = work[:M * K // 2].view(M, K // 2).cpu().numpy()
        off = (M * K // 2 + 255) // 256 * 256
        xs = work[off:off + 4 * M].view(torch.float32).cpu().numpy()
        rows = np.unique(np.concatenate([np.arange(5), np.arange(M - 5, M),
                                         np.random.default_rng(M).integers(0, M, 64)]))
        Y_ref = oracle.w4a4_gemm(xq[rows], xs[rows], Wq.cpu().numpy(), ws.cpu().numpy(), None, epi)
        acc.check_outputs(Yn[rows].float().cpu().numpy(), Y_ref, True, f"noalloc M={M} K={K}")


def test_noalloc_linear_rejects_rows_beyond_the_array(qv, dev):
    M, K, N = 16353, 4096, 128
    X = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    Wq = torch.zeros((N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.ones((N,), dtype=torch.float32, device=dev)
    Y = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
    with pytest.raises(qv.QVError, match="QV_ERR_WORKSPACE"):
        qv.qv_w4a4_linear_noalloc(X, None, Wq, ws, None, Y)
    torch.cuda.synchronize()
    assert bool((Y == 0).all()), "a rejected call wrote its output"
