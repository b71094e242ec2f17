"""MI355X (gfx950) W4A16 AWQ linear forward.

The compute lives in libawq_mi355x.so (hand-written HIP kernels behind the C
ABI of include/awq.h); this package is its thin Python binding plus a
WQLinear module with the interface of the page "Predibase Lorax AWQ WQLinear"
(Signature, I/O Contract).
"""
from __future__ import annotations

from .binding import (  # noqa: F401
    AWQ_PATH_DECODE, AWQ_PATH_GENERIC, AWQ_PATH_PREFILL, AwqError, PATH_NAMES, abi_version,
    dense_gemv, dequant, gemm, gemm_plan, gemm_workspace_size, lib, status_string,
    SortedWeight, dequant_gidx, gather_rows, gemm_gidx, gemm_sorted, gidx_layout, prepare_gidx,
    sorted_workspace_size,
)


def _module_base():
    import torch
    return torch.nn.Module


class WQLinear(_module_base()):
    """4-bit weight-quantised linear layer (page "Predibase Lorax AWQ
    WQLinear", Description): the construction checks and shape derivation of
    that page, and a forward that flattens the input to 2-D, runs the fused
    GEMM + bias kernel, and restores the leading dimensions.  Inference only.
    """

    def __init__(self, w_bit, group_size, qweight, qzeros, scales, bias):
        super().__init__()
        if w_bit != 4:
            raise ValueError("only 4-bit weights are supported")
        self.w_bit = w_bit
        self.in_features = qweight.shape[0]
        self.out_features = qweight.shape[1] * 32 // w_bit
        self.group_size = group_size if group_size != -1 else self.in_features
        if self.in_features % self.group_size != 0:
            raise ValueError("in_features must be divisible by group_size")
        if self.out_features % (32 // w_bit) != 0:
            raise ValueError("out_features must be divisible by 8")
        self.register_buffer("qweight", qweight)
        self.register_buffer("qzeros", qzeros)
        self.register_buffer("scales", scales)
        self.register_buffer("bias", bias)

    @property
    def weight(self):
        """The packed qweight tensor, for layer-interface compatibility."""
        return self.qweight

    def forward(self, x):
        import torch
        with torch.no_grad():
            return gemm(x, self.qweight, self.qzeros, self.scales, self.bias,
                        group_size=self.group_size)
