"""Seeded synthetic inputs for the W4A16 linear forward.

This module only draws random numbers in the shapes and value distributions
of the workloads; it holds none of the method's arithmetic (no unpacking, no
dequantisation, no contraction), so both the CPU oracle side and the GPU side
of a test can take their inputs from it.

Packed words are drawn as uniformly random 32-bit patterns: that is exactly
eight independent uniform draws of a 4-bit value in 0..15 per word, whatever
order the nibbles are read in, so no packing code is needed here.

Draw order for one problem (numpy PCG64, ``default_rng(seed)``):
qweight (K, N/8), qzeros (G, N/8), scales (G, N), bias (N) if any, x (M, K).
Weights are therefore identical across an M sweep that shares a seed, and the
first rows of x agree between two sweeps points.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    Ms: tuple
    K: int
    N: int
    group_sizes: tuple
    seed: int
    scale_lo: float
    scale_hi: float
    bias: bool
    note: str = field(default="", compare=False)


# The seeded workloads: a tiny case, the two decode shapes of the ROCm
# skinny-GEMM dispatch (K=8192, N in {1280, 7168}), a fused-QKV prefill
# projection, an MLP down-projection, batches between decode and prefill
# at the larger decode shape, and one GPU's shard of the two tensor-parallel
# layers.
WORKLOADS = {
    "tiny_m4_k256_n128": Workload(
        "tiny_m4_k256_n128", (4,), 256, 128, (64,), 0, 0.002, 0.02, True,
        "tiny W4A16 linear"),
    "decode_k8192_n1280": Workload(
        "decode_k8192_n1280", (1,), 8192, 1280, (128,), 1, 0.001, 0.01, False,
        "decode skinny GEMV"),
    "decode_sweep_k8192_n7168": Workload(
        "decode_sweep_k8192_n7168", (1, 4, 8, 16), 8192, 7168, (128,), 2,
        0.001, 0.01, False, "decode batch sweep"),
    "prefill_qkv_m2048_k4096_n12288": Workload(
        "prefill_qkv_m2048_k4096_n12288", (2048,), 4096, 12288, (128,), 3,
        0.001, 0.01, True, "prefill fused-QKV projection"),
    "mlp_down_k14336_n4096": Workload(
        "mlp_down_k14336_n4096", (1, 16, 256, 1024, 4096), 14336, 4096,
        (128, -1), 4, 0.001, 0.01, False, "MLP down-projection M sweep"),
    "midm_k8192_n7168": Workload(
        "midm_k8192_n7168", (32, 64, 128), 8192, 7168, (128,), 5, 0.001, 0.01, False,
        "batches between decode and prefill"),
    # One GPU's share of an 8-way tensor-parallel layer: a column shard of the
    # fused-QKV projection (N / 8 output columns) and a row shard of the
    # down-projection (K / 8 input rows, 14 groups of 128).
    "tp8_col_shard_qkv_m2048_k4096_n1536": Workload(
        "tp8_col_shard_qkv_m2048_k4096_n1536", (2048,), 4096, 1536, (128,), 6, 0.001, 0.01,
        True, "8-way column shard of the fused-QKV projection"),
    "tp8_row_shard_down_k1792_n4096": Workload(
        "tp8_row_shard_down_k1792_n4096", (1, 16, 256, 1024, 4096), 1792, 4096, (128,), 7,
        0.001, 0.01, False, "8-way row shard of the MLP down-projection"),
}


def num_groups(K: int, group_size: int) -> int:
    g = K if group_size == -1 else group_size
    return K // g


def make_inputs(M, K, N, group_size, seed, scale_lo=0.001, scale_hi=0.01,
                bias=False):
    """Draw one problem.  Returns a dict of numpy arrays:
    x (M, K) float16, qweight (K, N//8) int32, qzeros (G, N//8) int32,
    scales (G, N) float16, bias (N,) float16 or None."""
    G = num_groups(K, group_size)
    rng = np.random.default_rng(seed)
    qweight = rng.integers(0, 2 ** 32, size=(K, N // 8), dtype=np.uint32).view(np.int32)
    qzeros = rng.integers(0, 2 ** 32, size=(G, N // 8), dtype=np.uint32).view(np.int32)
    scales = rng.uniform(scale_lo, scale_hi, size=(G, N)).astype(np.float16)
    b = (rng.standard_normal(N) * 0.1).astype(np.float16) if bias else None
    x = rng.standard_normal((M, K)).astype(np.float16)
    return {"x": x, "qweight": qweight, "qzeros": qzeros, "scales": scales,
            "bias": b, "group_size": group_size}


def workload_inputs(name, M, group_size=None):
    """Inputs of a named workload at batch M (and group size, for the
    workload run at two group sizes)."""
    w = WORKLOADS[name]
    if M not in w.Ms:
        raise ValueError(f"M={M} is not a point of {name}")
    g = w.group_sizes[0] if group_size is None else group_size
    if g not in w.group_sizes:
        raise ValueError(f"group_size={g} is not a point of {name}")
    return make_inputs(M, w.K, w.N, g, w.seed, w.scale_lo, w.scale_hi, w.bias)


def act_order_g_idx(K, group_size, seed):
    """Row-to-group map of an activation-ordered quantisation: the K input
    rows are visited in a seeded random order and each run of group_size
    consecutive visited rows forms one group, so every group holds exactly
    group_size rows scattered over the input.  int32 (K,)."""
    if group_size <= 0 or K % group_size:
        raise ValueError("K must be a positive multiple of group_size")
    rng = np.random.default_rng(seed)
    order = rng.permutation(K)
    g_idx = np.empty(K, dtype=np.int32)
    g_idx[order] = np.arange(K, dtype=np.int64) // group_size
    return g_idx


def random_g_idx(K, G, seed):
    """Row-to-group map with independent uniform entries in [0, G): groups
    of unequal sizes, some possibly empty.  int32 (K,)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, G, size=K, dtype=np.int64).astype(np.int32)
