"""MI355X (gfx950) W4A16 AWQ linear forward.

The compute lives in libawq_mi355x.so (hand-written HIP kernels behind the C
ABI of include/awq.h); this package is its thin Python binding plus a
WQLinear module with the interface of the page "Predibase Lorax AWQ WQLinear"
(Signature, I/O Contract), and WQLinearGidx for weights under a row-to-group
map.
"""
from __future__ import annotations

from .binding import (  # noqa: F401
    AWQ_PATH_DECODE, AWQ_PATH_GENERIC, AWQ_PATH_PREFILL, AwqError, PATH_NAMES, abi_version,
    dense_gemv, dequant, gemm, gemm_plan, gemm_workspace_size, lib, status_string,
    SortedWeight, dequant_gidx, gather_rows, gemm_gidx, gemm_sorted, gidx_layout, prepare_gidx,
    sorted_workspace_size, get_option, options, set_option, gemm_noalloc,
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


class WQLinearGidx(_module_base()):
    """The same layer for weights whose rows map to groups through g_idx
    (the row-to-group map of the GPTQ tuple on the page "Predibase Lorax
    Linear Layer Factory", Description), with the packing of qweight and
    qzeros unchanged.  The weight is rebuilt once, at construction, as a
    grouped weight with its rows sorted by group (prepare_gidx); forward
    brings the columns of x into the same order and runs the grouped
    kernels (gemm_sorted).  Inference only.
    """

    def __init__(self, w_bit, qweight, qzeros, scales, g_idx, bias):
        super().__init__()
        if w_bit != 4:
            raise ValueError("only 4-bit weights are supported")
        self.w_bit = w_bit
        self.in_features = qweight.shape[0]
        self.out_features = qweight.shape[1] * 32 // w_bit
        self.num_groups = scales.shape[0]
        w = prepare_gidx(qweight, qzeros, scales, g_idx)
        self.block_rows = w.block_rows
        self.register_buffer("qweight", w.qweight)
        self.register_buffer("qzeros", w.qzeros)
        self.register_buffer("scales", w.scales)
        self.register_buffer("perm", w.perm)
        self.register_buffer("bias", bias)

    def forward(self, x):
        import torch
        w = SortedWeight(self.qweight, self.qzeros, self.scales, self.perm, self.block_rows,
                         self.in_features)
        with torch.no_grad():
            return gemm_sorted(x, w, self.bias)
