"""The GEMM that quantizes its own output for the next layer (qv_w4a4_gemm_requant): the MLP's
fc1 -> GELU -> bf16 -> width-N rotation -> smoothing -> int4 step in one launch.

Checked against the two-call form (qv_w4a4_gemm, then qv_hadamard_smooth_quant on its output) bit
for bit -- outputs, next-layer codes and scales -- and against the oracle stage-wise: the output
against the oracle's dequantization of the GPU's codes, the next-layer codes and scales against the
oracle's rotate-quantize of the GPU's output rows.  At the MLP workload's full size (mlp_24frames,
M = 32976) the fused chain equals the unfused chain bit for bit and sampled rows of fc2's input codes
match the oracle's chain end to end.  Sources: page "十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com),
训练后量化（PTQ）, 预全局旋转 and 后局部平滑."""
import numpy as np
import pytest

import acceptance as acc
from guard import check_codes_guard, check_guard, guarded_codes, guarded_output
import oracle
from bit_ptq_reconstruction_amd import configs, synth, workload

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


def bf16_host(t):
    return t.float().cpu().numpy()


def prepare(qv, dev, M, K, N, seed, smooth_next):
    """Seeded bf16 input quantized on the GPU, packed weights, and the next layer's factors."""
    X = synth.vggt_activations(M, K, seed=seed, dtype="bf16")
    W = synth.weights(N, K, seed=seed + 1)
    s, inv = oracle.smoothing(oracle.rotate(X[:min(M, synth.FRAME_TOKENS)], oracle.ROT_FWHT),
                              oracle.rotate(W, oracle.ROT_FWHT), 0.5)
    Xd = torch.from_numpy(X).to(dev).to(torch.bfloat16)
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((N,), dtype=torch.float32, device=dev)
    qv.qv_pack_weights(torch.from_numpy(W).to(dev), torch.from_numpy(s).to(dev), Wq, ws)
    Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty((M,), dtype=torch.float32, device=dev)
    qv.qv_hadamard_smooth_quant(Xd, torch.from_numpy(inv).to(dev), Xq, xs)
    inv_next = None
    if smooth_next:
        rng = np.random.default_rng(seed + 2)
        inv_next = torch.from_numpy(np.exp2(rng.uniform(-3, 3, N)).astype(np.float32)).to(dev)
    return Xq, xs, Wq, ws, inv_next


@pytest.mark.parametrize("M,K,N,epi,bias,smooth,pad", [
    (1, 1024, 4096, 1, False, True, 0),
    (129, 1024, 1024, 0, True, True, 0),      # a second stripe of one row
    (2749, 1024, 4096, 1, False, True, 0),    # two frames and one row: ragged last stripe
    (1374, 4096, 1024, 0, False, False, 0),   # width-4096 input, next width 1024
    (300, 1024, 4096, 1, True, True, 64),     # padded output rows
    (640, 1024, 1024, 1, False, False, 0),    # whole stripes only
])
def test_requant_equals_two_calls_and_oracle(qv, dev, M, K, N, epi, bias, smooth, pad):
    label = f"requant M={M} K={K} N={N} epi={epi} bias={bias} smooth={smooth} pad={pad}"
    print(label, flush=True)
    Xq, xs, Wq, ws, inv_next = prepare(qv, dev, M, K, N, 40 + M, smooth)
    b = torch.from_numpy(np.random.default_rng(M).standard_normal(N).astype(np.float32)).to(dev) if bias else None

    fullY, Y = guarded_output(M, N, torch.bfloat16, dev, ldy_pad=pad)
    qfull, q, sfull, s = guarded_codes(M, N // 2, 0, dev)
    work = torch.full((qv.qv_w4a4_gemm_requant_workspace_size(M),), 0x5A, dtype=torch.uint8, device=dev)
    qv.qv_w4a4_gemm_requant(Xq, xs, Wq, ws, b, Y, inv_next, q, s, work, epi)
    torch.cuda.synchronize()
    check_guard(fullY, M, N, label)
    check_codes_guard(qfull, sfull, M, label=label)

    # the two-call form
    Y2 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qv.qv_w4a4_gemm(Xq, xs, Wq, ws, b, Y2, epi)
    q2 = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
    s2 = torch.empty((M,), dtype=torch.float32, device=dev)
    qv.qv_hadamard_smooth_quant(Y2, inv_next, q2, s2)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), f"{label}: outputs differ from qv_w4a4_gemm"
    assert torch.equal(q, q2), f"{label}: next-layer codes differ from qv_hadamard_smooth_quant"
    assert torch.equal(s.view(torch.int32), s2.view(torch.int32)), f"{label}: next-layer scales differ"

    # stage-wise against the oracle
    rows = np.unique(np.concatenate([np.arange(min(M, 6)), np.arange(max(0, M - 6), M),
                                     np.random.default_rng(M + 1).integers(0, M, min(M, 96))]))
    Yr = bf16_host(Y[torch.from_numpy(rows).to(dev)])
    Y_ref = oracle.w4a4_gemm(Xq.cpu().numpy()[rows], xs.cpu().numpy()[rows], Wq.cpu().numpy(), ws.cpu().numpy(),
                             None if b is None else b.cpu().numpy(), epi)
    acc.check_outputs(Yr, Y_ref, True, f"{label} outputs")
    mult = None if inv_next is None else inv_next.cpu().numpy()
    Xh = oracle.rotate(Yr, oracle.ROT_FWHT)
    q_ref, s_ref = oracle.quantize_rows(Xh, mult)
    t, tau, _, rel = acc.code_bounds(Yr, mult, Xh)
    rate = acc.check_codes(oracle.unpack_int4(q.cpu().numpy()[rows]), q_ref, t, tau, f"{label} next-layer codes")
    acc.check_scales(s.cpu().numpy()[rows], s_ref, rel, f"{label} next-layer scales")
    print(f"{label}: next-layer code mismatch {rate:.1e}", flush=True)


def test_requant_repeated_calls(qv, dev):
    """The stripe counters are cleared by every call: repeated calls, and a call on fewer rows in
    between, give identical results on the same buffers."""
    M, K, N = 1000, 1024, 4096
    Xq, xs, Wq, ws, inv_next = prepare(qv, dev, M, K, N, 77, True)
    work = torch.empty((qv.qv_w4a4_gemm_requant_workspace_size(M),), dtype=torch.uint8, device=dev)
    outs = []
    for it, m in enumerate((M, M, 130, M)):
        print(f"requant repeated call {it} M={m}", flush=True)
        Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
        q = torch.empty((m, N // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((m,), dtype=torch.float32, device=dev)
        qv.qv_w4a4_gemm_requant(Xq[:m], xs[:m], Wq, ws, None, Y, inv_next, q, s, work, 1)
        torch.cuda.synchronize()
        outs.append((Y.clone(), q.clone(), s.clone()))
    for Y, q, s in outs[1:]:
        m = Y.shape[0]
        assert torch.equal(Y.view(torch.int16), outs[0][0][:m].view(torch.int16))
        assert torch.equal(q, outs[0][1][:m]) and torch.equal(s, outs[0][2][:m])


def test_requant_full_size_mlp_chain(qv, dev):
    """mlp_24frames (M = 32976): the fused chain (fc1 quantizing fc2's input) equals the unfused
    chain bit for bit, and sampled rows of fc2's input codes match the oracle's chain."""
    import test_gpu_fullsize as fs

    wl = configs.WORKLOADS["mlp_24frames"]
    fc1, fc2 = wl.linears
    M = wl.M
    X = synth.vggt_activations_torch(M, fc1.K, fc1.x_seed, torch.bfloat16, dev)
    W1, W2 = synth.weights(fc1.N, fc1.K, fc1.w_seed), synth.weights(fc2.N, fc2.K, fc2.w_seed)
    X0 = fs.host(X[:synth.FRAME_TOKENS])
    L1, s1, inv1 = fs.prepare_layer(qv, dev, fc1, M, X, W1, X0, wl.out_dtype)
    Wc1, ws1, _ = fs.check_weights(L1, W1, s1, "requant/fc1")
    q0, xs0 = oracle.hadamard_smooth_quant(X0, inv1, oracle.ROT_FWHT)
    Wq1_o, ws1_o = oracle.pack_weights(W1, s1, oracle.ROT_FWHT)
    Y1_0 = synth.round_to_bf16(oracle.w4a4_gemm(q0, xs0, Wq1_o, ws1_o, None, fc1.epi))
    L2, s2, inv2 = fs.prepare_layer(qv, dev, fc2, M, L1.Y, W2, Y1_0, wl.out_dtype)

    # unfused chain
    workload.run_linear(qv, L1)
    workload.run_linear(qv, L2)
    torch.cuda.synchronize()
    Y1_u, q2_u, s2_u, Y2_u = L1.Y.clone(), L2.Xq.clone(), L2.xs.clone(), L2.Y.clone()
    # fused chain: rotate-quantize fc1's input, fc1 with fc2's quantization, fc2's GEMM
    for t in (L1.Y, L2.Xq, L2.xs, L2.Y):
        t.zero_()
    work = torch.empty((qv.qv_w4a4_gemm_requant_workspace_size(M),), dtype=torch.uint8, device=dev)
    print("requant full-size fused chain", flush=True)
    qv.qv_hadamard_smooth_quant(L1.X, L1.inv, L1.Xq, L1.xs)
    qv.qv_w4a4_gemm_requant(L1.Xq, L1.xs, L1.Wq, L1.ws, None, L1.Y, L2.inv, L2.Xq, L2.xs, work, fc1.epi)
    qv.qv_w4a4_gemm(L2.Xq, L2.xs, L2.Wq, L2.ws, None, L2.Y, fc2.epi)
    torch.cuda.synchronize()
    assert torch.equal(L1.Y.view(torch.int16), Y1_u.view(torch.int16)), "fc1 outputs differ"
    assert torch.equal(L2.Xq, q2_u) and torch.equal(L2.xs.view(torch.int32), s2_u.view(torch.int32)), \
        "fc2 input codes or scales differ from the unfused chain"
    assert torch.equal(L2.Y.view(torch.int16), Y2_u.view(torch.int16)), "fc2 outputs differ"

    # end to end against the oracle's chain on sampled rows (code bound widened by fc1's difference)
    rows = fs.sample_rows(M, 11)
    X_rows = fs.host(X[torch.from_numpy(rows).to(dev)])
    _, _, Y1_ref = fs.check_rows(L1, rows, X_rows, inv1, Wc1, ws1, "requant/fc1")
    Y1_ref = synth.round_to_bf16(Y1_ref)
    Y1_gpu = fs.host(L1.Y[torch.from_numpy(rows).to(dev)])
    dX = np.abs(Y1_gpu.astype(np.float64) - Y1_ref)
    Xh = oracle.rotate(Y1_ref, oracle.ROT_FWHT)
    q_ref, s_ref = oracle.quantize_rows(Xh, inv2)
    t, tau, _, rel = acc.code_bounds(Y1_ref, inv2, Xh, dX=dX)
    rate = acc.check_codes(oracle.unpack_int4(L2.Xq[torch.from_numpy(rows).to(dev)].cpu().numpy()), q_ref, t, tau,
                           "requant/fc2 input (chain)")
    print(f"requant chain: fc2 input code mismatch {rate:.1e} over {len(rows)} rows", flush=True)
