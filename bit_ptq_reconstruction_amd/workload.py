"""Device-resident state of a named workload and the two library calls of one online linear.

A layer holds what the online step reads and writes: its input activations X (bf16 or fp32
[M][K]), the activation-side smoothing multipliers 1/s ([K] fp32), the quantized weights (packed
int4, or int8 for the W8A8 variant) and their per-channel scales (prepared once, offline), the
code/scale buffers of the quantized activations and the output Y [M][N].  ``run_linear`` is the
online path: rotate-smooth-quantize, then the GEMM with its dequant (+GELU) epilogue, both on the
given stream.

Smoothing follows the method's calibration reading: the factors of a layer come from the first
frame (1374 rows) of that layer's own input activations and from its weights.  In the MLP chain
fc2's input is fc1's output, so fc2 is calibrated on fc1's output for frame 0.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import synth
from .configs import Linear, Workload


@dataclass
class Layer:
    lin: Linear
    block: int
    X: object      # [M][K] activations (None until a chain links it)
    inv: object    # [K] fp32, 1 / smoothing factor
    Wq: object     # [N][K/2] uint8 packed int4 (or [N][K] int8) weight codes
    ws: object     # [N] fp32 weight scales
    Xq: object     # [M][K/2] uint8 packed int4 (or [M][K] int8) activation codes
    xs: object     # [M] fp32 activation scales
    Y: object      # [M][N] output
    bits: int = 4  # 4: packed int4 codes (W4A4); 8: int8 codes (W8A8)
    group: int = 0  # > 0: group-wise scales over that many channels (ws [N][K/group], xs [M][K/group])


def torch_dtype(name: str):
    import torch

    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def seeds(wl: Workload, lin: Linear, block: int):
    """(activation seed, weight seed) of a linear in a given block."""
    if wl.blocks > 1:
        return lin.x_seed + 1000 * block, lin.w_seed + 1000 * block
    return lin.x_seed, lin.w_seed


def run_linear(qv, L: Layer, stream=None) -> None:
    """The online linear: rotate-smooth-quantize, then the GEMM with its epilogue (W4A4 or W8A8)."""
    if L.bits == 8:
        qv.qv_hadamard_smooth_quant8(L.X, L.inv, L.Xq, L.xs, stream)
        qv.qv_w8a8_gemm(L.Xq, L.xs, L.Wq, L.ws, None, L.Y, L.lin.epi, stream)
    elif L.group:
        qv.qv_hadamard_smooth_quant_grouped(L.X, L.inv, L.group, L.Xq, L.xs, stream)
        qv.qv_w4a4_gemm_grouped(L.Xq, L.xs, L.Wq, L.ws, None, L.Y, L.group, L.lin.epi, stream)
    else:
        qv.qv_hadamard_smooth_quant(L.X, L.inv, L.Xq, L.xs, stream)
        qv.qv_w4a4_gemm(L.Xq, L.xs, L.Wq, L.ws, None, L.Y, L.lin.epi, stream)


def build(qv, wl: Workload, device, share_outputs: bool = False, bits: int = 4, group: int = 0, inputs=None):
    """Allocate and prepare every layer of ``wl`` on ``device`` (timing inputs, seeded on device).

    ``inputs``: layers of an earlier ``build`` of the same workload whose activation tensors are
    reused (they are the same seeded draws), so a variant of a large workload holds no second copy.

    Activations are drawn per layer and per block.  With ``share_outputs`` the code/scale buffers
    and outputs are shared by the layers of equal shape across blocks (a 48-block stack would
    otherwise hold 48 copies of buffers that each step overwrites in order).  Weights are packed
    with ``qv_pack_weights`` (``qv_pack_weights8`` for ``bits=8``) after ``qv_smooth_calibrate`` on
    frame 0 of the layer's input.  ``group`` > 0 (4-bit codes) uses group-wise scales
    (``qv_pack_weights_grouped``, ``qv_hadamard_smooth_quant_grouped``).
    """
    import torch

    M = wl.M
    in_dt, out_dt = torch_dtype(wl.in_dtype), torch_dtype(wl.out_dtype)
    code_dt = torch.int8 if bits == 8 else torch.uint8
    row_codes = (lambda K: K) if bits == 8 else (lambda K: K // 2)
    shared = {}

    def buffers(lin):
        key = (lin.name, lin.K, lin.N)
        if share_outputs and key in shared:
            return shared[key]
        b = (torch.empty((M, row_codes(lin.K)), dtype=code_dt, device=device),
             torch.empty((M, lin.K // group) if group else (M,), dtype=torch.float32, device=device),
             torch.empty((M, lin.N), dtype=out_dt, device=device))
        shared[key] = b
        return b

    layers = []
    for blk in range(wl.blocks):
        prev = None
        for li, lin in enumerate(wl.linears):
            x_seed, w_seed = seeds(wl, lin, blk)
            chained = wl.chain_mlp and li > 0
            if chained:
                X = None
            elif inputs is not None:
                X = inputs[len(layers)].X
                assert X.shape == (M, lin.K) and X.dtype == in_dt
            else:
                X = synth.vggt_activations_torch(M, lin.K, x_seed, in_dt, device)
            W = synth.weights_torch(lin.N, lin.K, w_seed, device)
            s = torch.empty(lin.K, device=device)
            inv = torch.empty(lin.K, device=device)
            if chained:
                calib = frame0_output(qv, prev, device)
            else:
                calib = X[:synth.FRAME_TOKENS]
            qv.qv_smooth_calibrate(calib, W, s, inv, 0.5)
            Wq = torch.empty((lin.N, row_codes(lin.K)), dtype=code_dt, device=device)
            ws = torch.empty((lin.N, lin.K // group) if group else (lin.N,), dtype=torch.float32, device=device)
            if group:
                qv.qv_pack_weights_grouped(W, s, group, Wq, ws)
            else:
                (qv.qv_pack_weights8 if bits == 8 else qv.qv_pack_weights)(W, s, Wq, ws)
            del W
            Xq, xs, Y = buffers(lin)
            L = Layer(lin, blk, X, inv, Wq, ws, Xq, xs, Y, bits, group)
            if chained:
                L.X = prev.Y
            layers.append(L)
            prev = L
    torch.cuda.synchronize(device)
    return layers


def frame0_output(qv, L: Layer, device):
    """Output of layer ``L`` on the first frame of its input (calibration rows of the next layer)."""
    import torch

    F = min(synth.FRAME_TOKENS, L.X.shape[0])
    tmp = Layer(L.lin, L.block, L.X[:F], L.inv, L.Wq, L.ws,
                torch.empty((F, L.Xq.shape[1]), dtype=L.Xq.dtype, device=device),
                torch.empty((F,) + tuple(L.xs.shape[1:]), dtype=torch.float32, device=device),
                torch.empty((F, L.lin.N), dtype=L.Y.dtype, device=device), L.bits, L.group)
    run_linear(qv, tmp)
    return tmp.Y
