"""The Python binding checks every tensor before the C call (CPU only: each case fails in the
checks, so nothing reaches the library or the GPU).  The C ABI sees bare pointers, so an undersized
output, a mismatched operand or a strided code matrix can only be caught here."""
import pytest
import torch

import bit_ptq_reconstruction_amd as qv

M, K, N = 8, 1024, 128


def ok_gemm(**kw):
    a = dict(Xq=torch.zeros((M, K // 2), dtype=torch.uint8), xs=torch.ones(M), Wq=torch.zeros((N, K // 2), dtype=torch.uint8),
             ws=torch.ones(N), bias=None, Y=torch.empty((M, N)))
    a.update(kw)
    return a


def call_gemm(a):
    qv.qv_w4a4_gemm(a["Xq"], a["xs"], a["Wq"], a["ws"], a["bias"], a["Y"])


@pytest.mark.parametrize("change,match", [
    (dict(Y=torch.empty((M, N - 1))), "Y has shape"),
    (dict(Y=torch.empty((M + 1, N))), "Y has shape"),
    (dict(Wq=torch.zeros((N, K // 2 - 16), dtype=torch.uint8)), "Wq has shape"),
    (dict(xs=torch.ones(M - 1)), "x_scale has shape"),
    (dict(ws=torch.ones(N + 1)), "w_scale has shape"),
    (dict(bias=torch.ones(N - 1)), "bias has shape"),
    (dict(Xq=torch.zeros((M, K // 2), dtype=torch.int8)), "Xq has dtype"),
    (dict(xs=torch.ones(M, dtype=torch.float64)), "x_scale has dtype"),
    (dict(Y=torch.empty((M, N), dtype=torch.float16)), "Y has dtype"),
    (dict(Xq=torch.zeros((M, K), dtype=torch.uint8)[:, ::2]), "Xq must be contiguous"),
    (dict(Wq=torch.zeros((K // 2, N), dtype=torch.uint8).t()), "Wq must be contiguous"),
    (dict(Y=torch.empty((N, M)).t()), "unit column stride"),
    ({}, "GPU tensor"),  # shapes right, but host tensors
])
def test_gemm_operands_checked(change, match):
    with pytest.raises(ValueError, match=match):
        call_gemm(ok_gemm(**change))


def test_rotate_quant_operands_checked():
    X = torch.zeros((M, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="codes has shape"):
        qv.qv_hadamard_smooth_quant(X, None, torch.zeros((M, K // 2 - 1), dtype=torch.uint8), torch.ones(M))
    with pytest.raises(ValueError, match="scales has shape"):
        qv.qv_hadamard_smooth_quant(X, None, torch.zeros((M, K // 2), dtype=torch.uint8), torch.ones(M - 1))
    with pytest.raises(ValueError, match="multiplier has shape"):
        qv.qv_hadamard_smooth_quant(X, torch.ones(K // 2), torch.zeros((M, K // 2), dtype=torch.uint8), torch.ones(M))
    with pytest.raises(ValueError, match="X has dtype"):
        qv.qv_hadamard_smooth_quant(X.half(), None, torch.zeros((M, K // 2), dtype=torch.uint8), torch.ones(M))
    with pytest.raises(ValueError, match="codes has dtype"):   # int8 codes belong to the 8-bit call
        qv.qv_hadamard_smooth_quant(X, None, torch.zeros((M, K // 2), dtype=torch.int8), torch.ones(M))
    with pytest.raises(ValueError, match="codes has shape"):
        qv.qv_hadamard_smooth_quant8(X, None, torch.zeros((M, K // 2), dtype=torch.int8), torch.ones(M))
    with pytest.raises(ValueError, match="GPU tensor"):
        qv.qv_pack_weights(torch.zeros((N, K)), None, torch.zeros((N, K // 2), dtype=torch.uint8), torch.ones(N))
    # a padded row stride is allowed for the input (the library takes ldx); it fails on the device only
    Xp = torch.zeros((M, K + 64), dtype=torch.bfloat16)[:, :K]
    with pytest.raises(ValueError, match="GPU tensor"):
        qv.qv_hadamard_smooth_quant(Xp, None, torch.zeros((M, K // 2), dtype=torch.uint8), torch.ones(M))


def test_linear_workspace_and_grouped_checked():
    X = torch.zeros((M, K), dtype=torch.bfloat16)
    Wq = torch.zeros((N, K // 2), dtype=torch.uint8)
    need = qv.qv_w4a4_linear_workspace_size(M, K)
    with pytest.raises(ValueError, match="workspace holds"):
        qv.qv_w4a4_linear(X, None, Wq, torch.ones(N), None, torch.empty((M, N)), torch.zeros(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace is required"):
        qv.qv_w4a4_linear(X, None, Wq, torch.ones(N), None, torch.empty((M, N)), None)
    with pytest.raises(ValueError, match="GPU tensor"):
        qv.qv_w4a4_linear(X, None, Wq, torch.ones(N), None, torch.empty((M, N)), torch.zeros(need, dtype=torch.uint8))
    G = K // 128
    with pytest.raises(ValueError, match="x_scale has shape"):
        qv.qv_w4a4_gemm_grouped(torch.zeros((M, K // 2), dtype=torch.uint8), torch.ones(M), Wq, torch.ones((N, G)),
                                None, torch.empty((M, N)), 128)
    with pytest.raises(ValueError, match="scales has shape"):
        qv.qv_hadamard_smooth_quant_grouped(X, None, 256, torch.zeros((M, K // 2), dtype=torch.uint8),
                                            torch.ones((M, G)))
    with pytest.raises(ValueError, match="must be positive and divide"):
        qv.qv_hadamard_smooth_quant_grouped(X, None, 96, torch.zeros((M, K // 2), dtype=torch.uint8),
                                            torch.ones((M, G)))
    with pytest.raises(ValueError, match="Wq8 has dtype"):
        qv.qv_w8a8_linear(X, None, torch.zeros((N, K), dtype=torch.uint8), torch.ones(N), None, torch.empty((M, N)),
                          torch.zeros(qv.qv_w8a8_linear_workspace_size(M, K), dtype=torch.uint8))
