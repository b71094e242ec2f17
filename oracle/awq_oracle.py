"""CPU oracle for the AWQ-style W4A16 linear forward.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
definition that the GPU path is checked against.  Only the test suite, the
package smoke check and the CPU-baseline leg of the benchmark may import it;
the product path (the C-ABI library and its Python binding) never does, and
this module imports nothing from the product path.

Source: the wiki page "Predibase Lorax AWQ WQLinear" (sections Description,
I/O Contract, Usage Examples).  Readings of points the page leaves open:

* Packing: the page says qweight is int32 of shape (in_features,
  out_features // 8), each word holding eight four-bit values along the output
  dimension.  The order of the eight nibbles inside a word is not given; this
  oracle reads it as sequential, least-significant nibble first: bits
  [4j, 4j+3] of word (k, c) hold output column 8c + j.  Nibbles are unsigned.
* qzeros: "packed quantized zero points" with no shape given; read as int32
  (G, out_features // 8) packed exactly like qweight, G = in_features // group_size.
* scales: "per-group scale factors" with no shape/dtype given; read as float16
  (G, out_features).
* Groups: group_size consecutive input rows share one scale/zero row, so row k
  uses group k // group_size; group_size == -1 means one group of in_features.
* Dequantisation: w[k, n] = float16_RNE((q[k, n] - z[k//g, n]) * s[k//g, n]),
  one rounding of the exact product, no zero-point offset.
* Contraction: y = x . W (+ bias), evaluated in float64 (exact products of
  float16 values, float64 summation); bias added in float64.

Functions:
    validate(...)          -- the page's __init__ checks plus shape checks
    pack_int4 / unpack_int4
    dequant(...)           -- float16 (K, N) dequantised weight
    awq_linear_ref(...)    -- float64 forward, (*, K) -> (*, N)
    awq_linear_loops(...)  -- pure-Python triple loop, for tiny inputs only
    dense_linear_ref(...)  -- the unquantised float16 linear (baseline), float64
    dense_linear_loops     -- its pure-Python triple loop, for tiny inputs only

Row-to-group map (g_idx): the page "Predibase Lorax Linear Layer Factory"
(Description, the get_linear bullets) lists g_idx among the quantised
weight's components (the GPTQ tuple) and says no more about it.  Read here as
the plainest generalisation of the contiguous groups above: g_idx is an
integer vector of length in_features whose entry k names the scale/zero row
of input row k, so w[k, n] = float16_RNE((q[k, n] - z[g_idx[k], n]) *
s[g_idx[k], n]); g_idx[k] = k // group_size is the contiguous case.  The
packing of qweight and qzeros stays the one above.

    validate_gidx(...)     -- shape and range checks of a row-to-group map
    dequant_gidx(...)      -- float16 (K, N) dequantised weight under a map
    awq_linear_gidx_ref    -- float64 forward under a map
    awq_linear_gidx_loops  -- its pure-Python triple loop, for tiny inputs
    gidx_order(...)        -- stable sort of the rows by group (rows of each
                              group contiguous, ties in input order)

The unquantised linear follows the page "Predibase Lorax Linear Layer
Factory" (Description: FastLinear, a float16 F.linear whose weight is
(out_features, in_features); its ROCm variant sends single-token products at
in_features 8192 and out_features 1280 or 7168 to a custom skinny kernel):
y = x . w^T (+ bias).
"""
from __future__ import annotations

import numpy as np

W_BIT = 4
PACK = 32 // W_BIT  # eight nibbles per int32 word


def validate(w_bit, group_size, qweight_shape, qzeros_shape=None,
             scales_shape=None, bias_shape=None):
    """The construction checks of WQLinear (page "Predibase Lorax AWQ
    WQLinear", Description, the __init__ bullets), re-stated.

    Returns (K, N, g, G).  Raises ValueError on any violation.
    """
    if w_bit != 4:
        raise ValueError("only 4-bit weights are supported")
    if len(qweight_shape) != 2:
        raise ValueError("qweight must be 2-D")
    K = int(qweight_shape[0])
    N = int(qweight_shape[1]) * 32 // w_bit
    if K <= 0 or N <= 0:
        raise ValueError("empty weight")
    g = K if group_size == -1 else int(group_size)
    if g <= 0:
        raise ValueError("group_size must be positive or -1")
    if K % g != 0:
        raise ValueError("in_features must be divisible by group_size")
    if N % (32 // w_bit) != 0:
        raise ValueError("out_features must be divisible by 8")
    G = K // g
    if qzeros_shape is not None and tuple(qzeros_shape) != (G, N // PACK):
        raise ValueError(f"qzeros shape {tuple(qzeros_shape)} != {(G, N // PACK)}")
    if scales_shape is not None and tuple(scales_shape) != (G, N):
        raise ValueError(f"scales shape {tuple(scales_shape)} != {(G, N)}")
    if bias_shape is not None and tuple(bias_shape) != (N,):
        raise ValueError(f"bias shape {tuple(bias_shape)} != {(N,)}")
    return K, N, g, G


def pack_int4(q):
    """Pack integers 0..15 of shape (R, C), C % 8 == 0, into int32 (R, C//8):
    word (r, c) = sum_j q[r, 8c+j] << 4j, assembled as uint32 so that a value
    >= 8 in the top nibble does not overflow, then reinterpreted as int32."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[1] % PACK != 0:
        raise ValueError("pack_int4 needs a 2-D array whose width is a multiple of 8")
    if q.size and (q.min() < 0 or q.max() > 15):
        raise ValueError("pack_int4 values must lie in 0..15")
    R, C = q.shape
    words = np.zeros((R, C // PACK), dtype=np.uint64)
    for j in range(PACK):
        words |= q[:, j::PACK].astype(np.uint64) << np.uint64(4 * j)
    return words.astype(np.uint32).view(np.int32)


def unpack_int4(p):
    """Inverse of pack_int4: int32 (R, C) -> int64 (R, 8C) with
    out[r, 8c+j] = (uint32(p[r, c]) >> 4j) & 0xF."""
    p = np.asarray(p)
    if p.dtype != np.int32 or p.ndim != 2:
        raise ValueError("unpack_int4 needs a 2-D int32 array")
    u = p.view(np.uint32).astype(np.int64)
    R, C = u.shape
    out = np.empty((R, C * PACK), dtype=np.int64)
    for j in range(PACK):
        out[:, j::PACK] = (u >> (4 * j)) & 0xF
    return out


def dequant(qweight, qzeros, scales, group_size):
    """Group-wise dequantisation to float16 (K, N).

    q is unpacked from qweight, z from qzeros (row k//g), s from scales
    (row k//g); each weight is (q - z) * s formed exactly in float64 and
    rounded once to float16 (round to nearest even, subnormals kept).
    """
    scales = np.asarray(scales)
    K, N, g, G = validate(4, group_size, qweight.shape, qzeros.shape, scales.shape)
    q = unpack_int4(qweight)                       # (K, N)
    z = unpack_int4(qzeros)                        # (G, N)
    grp = np.arange(K) // g                        # group of each input row
    diff = (q - z[grp, :]).astype(np.float64)      # exact integer in [-15, 15]
    s = scales.astype(np.float64)[grp, :]          # exact float16 values
    with np.errstate(over="ignore"):                # |product| > 65504 -> inf, as IEEE
        return (diff * s).astype(np.float16)       # one rounding


def awq_linear_ref(x, qweight, qzeros, scales, bias, group_size):
    """Forward of WQLinear (page "Predibase Lorax AWQ WQLinear", Description,
    forward steps 1-3): flatten x to (M, K), contract with the dequantised
    weight, add the optional bias, restore the leading dimensions.

    Returns float64 of shape (*x.shape[:-1], N).
    """
    x = np.asarray(x)
    w = dequant(qweight, qzeros, scales, group_size)
    K, N = w.shape
    if x.shape[-1] != K:
        raise ValueError(f"input feature size {x.shape[-1]} != in_features {K}")
    lead = x.shape[:-1]
    x2 = x.reshape(-1, K).astype(np.float64)
    y = x2 @ w.astype(np.float64)
    if bias is not None:
        b = np.asarray(bias)
        if b.shape != (N,):
            raise ValueError("bias must have shape (out_features,)")
        y = y + b.astype(np.float64)[None, :]
    return y.reshape(*lead, N)


def awq_linear_loops(x, qweight, qzeros, scales, bias, group_size):
    """Pure-Python restatement for tiny inputs: every weight is unpacked from
    its word with shifts, dequantised with Python floats and accumulated in a
    plain loop.  Independent of the numpy code paths above."""
    M = len(x)
    K = len(qweight)
    N = len(qweight[0]) * PACK
    g = K if group_size == -1 else group_size
    y = [[0.0] * N for _ in range(M)]
    for n in range(N):
        c, j = divmod(n, PACK)
        for k in range(K):
            word = int(qweight[k][c]) & 0xFFFFFFFF
            q = (word >> (4 * j)) & 0xF
            zword = int(qzeros[k // g][c]) & 0xFFFFFFFF
            z = (zword >> (4 * j)) & 0xF
            s = float(scales[k // g][n])
            w = float(np.float16((q - z) * s))
            for m in range(M):
                y[m][n] += float(x[m][k]) * w
    if bias is not None:
        for m in range(M):
            for n in range(N):
                y[m][n] += float(bias[n])
    return np.array(y, dtype=np.float64)


def dense_linear_ref(x, w, bias):
    """The unquantised FastLinear forward (page "Predibase Lorax Linear Layer
    Factory", Description): F.linear(x, w, bias) = x . w^T + bias with w of
    shape (out_features, in_features), evaluated in float64 (exact products of
    float16 values).  Returns float64 of shape (*x.shape[:-1], N)."""
    x = np.asarray(x)
    w = np.asarray(w)
    N, K = w.shape
    if x.shape[-1] != K:
        raise ValueError(f"input feature size {x.shape[-1]} != in_features {K}")
    lead = x.shape[:-1]
    y = x.reshape(-1, K).astype(np.float64) @ w.astype(np.float64).T
    if bias is not None:
        b = np.asarray(bias)
        if b.shape != (N,):
            raise ValueError("bias must have shape (out_features,)")
        y = y + b.astype(np.float64)[None, :]
    return y.reshape(*lead, N)


def dense_linear_loops(x, w, bias):
    """Pure-Python restatement of dense_linear_ref for tiny inputs."""
    M, K, N = len(x), len(x[0]), len(w)
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(x[m][k]) * float(w[n][k])
            y[m][n] = acc + (float(bias[n]) if bias is not None else 0.0)
    return np.array(y, dtype=np.float64)


def validate_gidx(g_idx, K, G):
    """A row-to-group map for K input rows and G scale/zero rows: integer
    vector of shape (K,) with every entry in [0, G).  Returns it as int64."""
    g_idx = np.asarray(g_idx)
    if g_idx.shape != (K,):
        raise ValueError(f"g_idx shape {g_idx.shape} != {(K,)}")
    if g_idx.size and not np.issubdtype(g_idx.dtype, np.integer):
        raise ValueError("g_idx must hold integers")
    g_idx = g_idx.astype(np.int64)
    if G <= 0:
        raise ValueError("need at least one group")
    if g_idx.size and (g_idx.min() < 0 or g_idx.max() >= G):
        raise ValueError("g_idx entries must lie in [0, G)")
    return g_idx


def dequant_gidx(qweight, qzeros, scales, g_idx):
    """Dequantisation with a row-to-group map: input row k takes zero row
    g_idx[k] of qzeros and scale row g_idx[k] of scales; each weight is
    (q - z) * s formed exactly in float64 and rounded once to float16."""
    scales = np.asarray(scales)
    qzeros = np.asarray(qzeros)
    if scales.ndim != 2:
        raise ValueError("scales must be 2-D")
    G = scales.shape[0]
    K = int(qweight.shape[0])
    N = int(qweight.shape[1]) * PACK
    if K <= 0 or N <= 0:
        raise ValueError("empty weight")
    if tuple(qzeros.shape) != (G, N // PACK) or tuple(scales.shape) != (G, N):
        raise ValueError("qzeros must be (G, N/8) and scales (G, N)")
    grp = validate_gidx(g_idx, K, G)
    q = unpack_int4(qweight)                       # (K, N)
    z = unpack_int4(qzeros)                        # (G, N)
    diff = (q - z[grp, :]).astype(np.float64)      # exact integer in [-15, 15]
    s = scales.astype(np.float64)[grp, :]
    with np.errstate(over="ignore"):
        return (diff * s).astype(np.float16)       # one rounding


def awq_linear_gidx_ref(x, qweight, qzeros, scales, g_idx, bias):
    """Forward under a row-to-group map: y = x . dequant_gidx(...) (+ bias)
    in float64, (*, K) -> (*, N)."""
    x = np.asarray(x)
    w = dequant_gidx(qweight, qzeros, scales, g_idx)
    K, N = w.shape
    if x.shape[-1] != K:
        raise ValueError(f"input feature size {x.shape[-1]} != in_features {K}")
    lead = x.shape[:-1]
    y = x.reshape(-1, K).astype(np.float64) @ w.astype(np.float64)
    if bias is not None:
        b = np.asarray(bias)
        if b.shape != (N,):
            raise ValueError("bias must have shape (out_features,)")
        y = y + b.astype(np.float64)[None, :]
    return y.reshape(*lead, N)


def awq_linear_gidx_loops(x, qweight, qzeros, scales, g_idx, bias):
    """Pure-Python restatement of awq_linear_gidx_ref for tiny inputs: the
    group of row k is looked up in g_idx, nibbles are taken with shifts."""
    M = len(x)
    K = len(qweight)
    N = len(qweight[0]) * PACK
    y = [[0.0] * N for _ in range(M)]
    for n in range(N):
        c, j = divmod(n, PACK)
        for k in range(K):
            gk = int(g_idx[k])
            q = ((int(qweight[k][c]) & 0xFFFFFFFF) >> (4 * j)) & 0xF
            z = ((int(qzeros[gk][c]) & 0xFFFFFFFF) >> (4 * j)) & 0xF
            w = float(np.float16((q - z) * float(scales[gk][n])))
            for m in range(M):
                y[m][n] += float(x[m][k]) * w
    if bias is not None:
        for m in range(M):
            for n in range(N):
                y[m][n] += float(bias[n])
    return np.array(y, dtype=np.float64)


def gidx_order(g_idx, G):
    """Rows sorted by group, stably: perm[j] is the input row placed j-th,
    so the rows of group 0 come first in increasing input order, then those
    of group 1, and so on.  Also returns the number of rows of each group."""
    grp = validate_gidx(g_idx, len(np.asarray(g_idx)), G)
    perm = np.argsort(grp, kind="stable")
    counts = np.bincount(grp, minlength=G)
    return perm.astype(np.int64), counts.astype(np.int64)
