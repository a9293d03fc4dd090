"""Named VGGT-shaped workloads (shapes and seeds only).

Every workload is a list of linears (name, K, N, epilogue, input dtype) over M = 1374 x frames
token rows; K is also the Hadamard width.  The block's four linears are qkv 1024->3072,
proj 1024->1024, fc1 1024->4096 with GELU, fc2 4096->1024 (its input is rotated at width 4096).
"""
from __future__ import annotations

from dataclasses import dataclass, field

from .synth import FRAME_TOKENS

EPI_NONE = 0
EPI_GELU = 1


@dataclass(frozen=True)
class Linear:
    name: str
    K: int
    N: int
    epi: int = EPI_NONE
    x_seed: int = 0
    w_seed: int = 1


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    frames: int
    in_dtype: str  # "fp32" or "bf16"
    out_dtype: str  # "fp32" or "bf16"
    linears: tuple = field(default_factory=tuple)
    blocks: int = 1
    chain_mlp: bool = False  # fc2 consumes fc1's (GELU, bf16) output

    @property
    def M(self) -> int:
        return FRAME_TOKENS * self.frames


def block_linears(block: int = 0):
    names = [("qkv", 1024, 3072, EPI_NONE), ("proj", 1024, 1024, EPI_NONE),
             ("fc1", 1024, 4096, EPI_GELU), ("fc2", 4096, 1024, EPI_NONE)]
    return tuple(Linear(n, K, N, e, x_seed=1000 * block + i, w_seed=500000 + 1000 * block + i)
                 for i, (n, K, N, e) in enumerate(names))


WORKLOADS = {
    "single_1frame": Workload(
        "single_1frame", "one 1024->1024 W4A4 linear, 1 frame (M=1374), fp32 in/out",
        frames=1, in_dtype="fp32", out_dtype="fp32",
        linears=(Linear("linear", 1024, 1024, EPI_NONE, 0, 1),)),
    "qkv_8frames": Workload(
        "qkv_8frames", "qkv projection 1024->3072, 8 frames (M=10992), bf16",
        frames=8, in_dtype="bf16", out_dtype="bf16",
        linears=(Linear("qkv", 1024, 3072, EPI_NONE, 0, 1),)),
    "mlp_24frames": Workload(
        "mlp_24frames", "fc1 1024->4096 + GELU -> bf16 -> width-4096 rotate-quantize -> fc2 4096->1024, "
        "24 frames (M=32976), bf16 (two-call chain; qv_w4a4_gemm_requant fuses the requantization into fc1)",
        frames=24, in_dtype="bf16", out_dtype="bf16",
        linears=(Linear("fc1", 1024, 4096, EPI_GELU, 0, 1), Linear("fc2", 4096, 1024, EPI_NONE, 0, 2)),
        chain_mlp=True),
    "block_32frames": Workload(
        "block_32frames", "the four linears of one block (qkv, proj, fc1+GELU, fc2), 32 frames "
        "(M=43968), bf16", frames=32, in_dtype="bf16", out_dtype="bf16",
        linears=block_linears(0)),
    "stack48_100frames": Workload(
        "stack48_100frames", "48-block linear stack (192 linears), 100 frames (M=137400), bf16",
        frames=100, in_dtype="bf16", out_dtype="bf16", linears=block_linears(0), blocks=48),
}
