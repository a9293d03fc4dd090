"""Seeded synthetic VGGT-shaped inputs.  No quantization, rotation or contraction happens here.

The token layout follows the VGGT description on the QuantVGGT method page ("十亿参数的三维重建模型，
能塞进手机吗？", gslzct.com, section 视觉几何基础 Transformer（VGGT）): every frame carries one camera
token and four register tokens in front of its image-patch tokens, and section 双平滑细粒度量化 >
观察 1 says these first five tokens carry the heavy-tailed outliers.  A frame here is 5 special rows
followed by 37 x 37 = 1369 patch rows (1374 rows), patch rows ~ N(0, 1), special rows x20, and eight
outlier channels x50 shared by every row of a layer.  Weights are N(0, 0.02^2).

Two generators exist:
  * ``vggt_activations`` / ``weights``: numpy PCG64, host arrays, used for parity (both the HIP
    path and the oracle receive the same arrays);
  * ``vggt_activations_torch`` / ``weights_torch``: the same recipe drawn on the device with a
    seeded torch generator, used for timing only (values differ from the numpy stream).
"""
from __future__ import annotations

import numpy as np

FRAME_TOKENS = 1374
SPECIAL_TOKENS = 5
SPECIAL_SCALE = 20.0
OUTLIER_CHANNELS = 8
OUTLIER_SCALE = 50.0
WEIGHT_STD = 0.02


def outlier_channels(K: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 0xC01])
    return np.sort(rng.choice(K, size=min(OUTLIER_CHANNELS, K), replace=False))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), returned as fp32 (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def vggt_activations(M: int, K: int, seed: int, dtype: str = "fp32", first_row: int = 0) -> np.ndarray:
    """Rows [first_row, first_row + M) of the seeded activation stream, as fp32 values.

    Each frame is drawn from its own generator, so any row range can be regenerated alone.
    ``dtype='bf16'`` rounds the values to bf16 (still returned as fp32)."""
    cols = outlier_channels(K, seed)
    out = np.empty((M, K), dtype=np.float32)
    r = first_row
    end = first_row + M
    while r < end:
        f = r // FRAME_TOKENS
        lo = r - f * FRAME_TOKENS
        hi = min(FRAME_TOKENS, end - f * FRAME_TOKENS)
        rng = np.random.default_rng([seed, f + 1])
        block = rng.standard_normal((FRAME_TOKENS, K))
        block[:SPECIAL_TOKENS] *= SPECIAL_SCALE
        block[:, cols] *= OUTLIER_SCALE
        out[r - first_row:r - first_row + (hi - lo)] = block[lo:hi].astype(np.float32)
        r += hi - lo
    if dtype == "bf16":
        out = round_to_bf16(out)
    elif dtype != "fp32":
        raise ValueError(dtype)
    return out


def weights(N: int, K: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 0x57])
    return (WEIGHT_STD * rng.standard_normal((N, K))).astype(np.float32)


def vggt_activations_torch(M: int, K: int, seed: int, dtype, device):
    """The same recipe drawn on the device (timing inputs; not bit-identical to the numpy stream)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    rows = torch.arange(M, device=device) % FRAME_TOKENS
    x[rows < SPECIAL_TOKENS] *= SPECIAL_SCALE
    cols = torch.as_tensor(outlier_channels(K, seed), device=device)
    x[:, cols] *= OUTLIER_SCALE
    return x.to(dtype)


def weights_torch(N: int, K: int, seed: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) + 0x57)
    return WEIGHT_STD * torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
