"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Bar: awq_dequant bit-exact; awq_gemm within |gpu - ref| <= 1e-2 + 1e-2*|ref|
elementwise against the float64 oracle; exact equality where the arithmetic
is exact (one-hot rows, q == z, group_size -1 against K, golden examples).
Inputs come from the seeded generator in awq_inputs; expected values come
only from the oracle or the hand-computed golden file.
"""
import functools
import os
import sys

import numpy as np
import pytest

import awq_inputs
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_weight_quantized_awq_amd as awq  # noqa: E402
from bit_weight_quantized_awq_amd import binding  # noqa: E402

ATOL = 1e-2
RTOL = 1e-2
DEV = "cuda:0"


def say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert "gfx950" in name, f"expected gfx950, got {name}"
    # The HIP library must be what runs: loading it is the first step.
    awq.lib()
    yield


def to_dev(p):
    d = {k: (torch.from_numpy(np.ascontiguousarray(v)).to(DEV) if isinstance(v, np.ndarray)
             else v) for k, v in p.items()}
    return d


ZERO_REGION = 4 * 65536 * 16   # accumulator region of a decode workspace


def assert_within_tol(gpu, ref, what):
    gpu = gpu.astype(np.float64)
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {tuple(i)}: "
            f"gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r}; max err {err.max():.3e}")


def run_gemm(d, path=None, M=None, opts=None):
    """awq_gemm on device inputs d; path forces a kernel family, opts sets
    further planner overrides (awq.options) for the call only."""
    x = d["x"] if M is None else d["x"][:M]
    opts = dict(opts or {})
    if path is not None:
        opts["force_path"] = path
    with awq.options(**opts):
        y = awq.gemm(x, d["qweight"], d["qzeros"], d["scales"], d["bias"], d["group_size"])
        torch.cuda.synchronize()
    return y.cpu().numpy()


@functools.lru_cache(maxsize=8)
def cached_problem(name, Mmax, g):
    p = awq_inputs.workload_inputs(name, Mmax, g)
    w = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    return p, w


# ------------------------------------------------------------------ golden
def load_golden():
    sys.path.insert(0, os.path.dirname(__file__))
    from test_oracle import GOLDEN_CASES
    return GOLDEN_CASES


@pytest.mark.parametrize("idx", range(4))
def test_golden_examples(idx):
    ex = load_golden()[idx]
    say(f"golden {ex['name']} generic + dequant")
    d = to_dev(dict(x=ex["x"], qweight=ex["qweight"], qzeros=ex["qzeros"], scales=ex["scales"],
                    bias=ex["bias"], group_size=ex["g"]))
    w = awq.dequant(d["qweight"], d["qzeros"], d["scales"], ex["g"]).cpu().numpy()
    np.testing.assert_array_equal(w.view(np.uint16), ex["w_bits"])
    y = run_gemm(d)
    np.testing.assert_array_equal(y.astype(np.float64), ex["y"].astype(np.float16).astype(np.float64))


# ----------------------------------------------------------------- dequant
DEQUANT_CASES = [
    ("tiny_m4_k256_n128", 4, 64),
    ("decode_k8192_n1280", 1, 128),
    ("decode_sweep_k8192_n7168", 1, 128),
    ("prefill_qkv_m2048_k4096_n12288", 2048, 128),
    ("mlp_down_k14336_n4096", 1, 128),
    ("mlp_down_k14336_n4096", 1, -1),
]


@pytest.mark.parametrize("name,M,g", DEQUANT_CASES)
def test_dequant_bit_exact(name, M, g):
    say(f"awq_dequant {name} g={g}")
    p = awq_inputs.workload_inputs(name, M, g)
    d = to_dev(p)
    w = awq.dequant(d["qweight"], d["qzeros"], d["scales"], g).cpu().numpy()
    ref = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    np.testing.assert_array_equal(w.view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("K,N,g", [(8, 8, 1), (24, 40, 3), (96, 24, -1), (64, 136, 16)])
def test_dequant_odd_shapes_and_signed_scales(K, N, g):
    say(f"awq_dequant odd K={K} N={N} g={g}")
    p = awq_inputs.make_inputs(1, K, N, g, seed=K + N, scale_lo=-4.0, scale_hi=4.0)
    d = to_dev(p)
    w = awq.dequant(d["qweight"], d["qzeros"], d["scales"], g).cpu().numpy()
    ref = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    np.testing.assert_array_equal(w.view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("g", [128, -1])
def test_dequant_streamed_output_sampled_groups(g):
    """A W larger than the last-level cache (K = 8192, N = 14336: 235 MB)
    takes the nontemporal-store form.  Each group of rows depends only on
    its own packed rows and its zero/scale row, so whole sampled groups
    (first, last and two seeded ones) are checked bit for bit against the
    oracle on just those rows."""
    K, N = 8192, 14336
    say(f"awq_dequant streamed K={K} N={N} g={g}")
    rng = np.random.default_rng(21)
    qw = rng.integers(0, 2 ** 32, size=(K, N // 8), dtype=np.uint32).view(np.int32)
    gs = K if g == -1 else g
    G = K // gs
    qz = rng.integers(0, 2 ** 32, size=(G, N // 8), dtype=np.uint32).view(np.int32)
    sc = rng.uniform(-0.02, 0.02, size=(G, N)).astype(np.float16)
    w = awq.dequant(torch.from_numpy(qw).to(DEV), torch.from_numpy(qz).to(DEV),
                    torch.from_numpy(sc).to(DEV), g)
    torch.cuda.synchronize()
    for grp in sorted({0, G - 1, int(rng.integers(0, G)), int(rng.integers(0, G))}):
        rows = slice(grp * gs, (grp + 1) * gs) if g != -1 else slice(0, 256)
        got = w[rows].cpu().numpy()
        ref = oracle.dequant(qw[rows], qz[grp:grp + 1], sc[grp:grp + 1],
                             got.shape[0] if g == -1 else g)
        np.testing.assert_array_equal(got.view(np.uint16), ref.view(np.uint16))


def _offset_copy(a, words):
    """A contiguous device copy of `a` that starts `words` elements into a
    larger buffer (so it is not 16-byte aligned)."""
    t = torch.from_numpy(np.ascontiguousarray(a)).reshape(-1)
    buf = torch.zeros(t.numel() + words, dtype=t.dtype)
    buf[words:] = t
    return buf.to(DEV)[words:].view(a.shape)


@pytest.mark.parametrize("qw_off,sc_off", [(0, 0), (1, 0), (0, 1), (3, 5)])
def test_dequant_alignment_forms(qw_off, sc_off):
    """awq_dequant takes its widest form (4 words per thread) only for 16-byte
    aligned operands; offset operands take the narrower forms, bit for bit
    the same."""
    say(f"awq_dequant alignment qweight+{qw_off} scales+{sc_off}")
    K, N, g = 256, 512, 64
    p = awq_inputs.make_inputs(1, K, N, g, seed=11, scale_lo=-2.0, scale_hi=2.0)
    qw = _offset_copy(p["qweight"], qw_off)
    qz = _offset_copy(p["qzeros"], qw_off)
    sc = _offset_copy(p["scales"], sc_off)
    w = awq.dequant(qw, qz, sc, g).cpu().numpy()
    ref = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    np.testing.assert_array_equal(w.view(np.uint16), ref.view(np.uint16))


# ---------------------------------------------------------- config parity
GEMM_CASES = [
    ("tiny_m4_k256_n128", 4, 4, 64),
    ("decode_k8192_n1280", 1, 1, 128),
    ("decode_sweep_k8192_n7168", 16, 1, 128),
    ("decode_sweep_k8192_n7168", 16, 4, 128),
    ("decode_sweep_k8192_n7168", 16, 8, 128),
    ("decode_sweep_k8192_n7168", 16, 16, 128),
    ("mlp_down_k14336_n4096", 4096, 1, 128),
    ("mlp_down_k14336_n4096", 4096, 16, 128),
    ("mlp_down_k14336_n4096", 4096, 256, 128),
    ("mlp_down_k14336_n4096", 4096, 1024, 128),
    ("mlp_down_k14336_n4096", 4096, 4096, 128),
    ("mlp_down_k14336_n4096", 4096, 1, -1),
    ("mlp_down_k14336_n4096", 4096, 16, -1),
    ("mlp_down_k14336_n4096", 4096, 256, -1),
    ("mlp_down_k14336_n4096", 4096, 1024, -1),
    ("mlp_down_k14336_n4096", 4096, 4096, -1),
    ("prefill_qkv_m2048_k4096_n12288", 2048, 2048, 128),
    ("midm_k8192_n7168", 128, 32, 128),
    ("midm_k8192_n7168", 128, 64, 128),
    ("midm_k8192_n7168", 128, 128, 128),
]


@pytest.mark.parametrize("name,Mmax,M,g", GEMM_CASES)
def test_gemm_config_parity(name, Mmax, M, g):
    """Every workload point, every output element, against the oracle's
    forward (oracle.awq_linear_ref: float16 dequantisation, float64
    contraction and bias)."""
    say(f"awq_gemm {name} M={M} g={g}")
    p = awq_inputs.workload_inputs(name, Mmax, g)
    d = to_dev(p)
    K, N = p["qweight"].shape[0], p["qweight"].shape[1] * 8
    path, _ = awq.gemm_plan(M, K, N, g, d["x"].data_ptr(), d["scales"].data_ptr())
    # Up to 16 rows the decode kernel; 17-32 rows (here M = 32 of the 29 MB
    # weight) its two-block form; above, the prefill kernel.
    expect_path = binding.AWQ_PATH_DECODE if M <= 32 else binding.AWQ_PATH_PREFILL
    assert path == expect_path
    y = run_gemm(d, M=M)
    del d
    ref = oracle.awq_linear_ref(p["x"][:M], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    assert ref.shape == y.shape == (M, N)
    assert_within_tol(y, ref, f"{name} M={M} g={g}")


@pytest.mark.parametrize("name,Mmax,M", [
    ("tp8_col_shard_qkv_m2048_k4096_n1536", 2048, 2048),
    ("tp8_row_shard_down_k1792_n4096", 4096, 1),
    ("tp8_row_shard_down_k1792_n4096", 4096, 16),
    ("tp8_row_shard_down_k1792_n4096", 4096, 256),
    ("tp8_row_shard_down_k1792_n4096", 4096, 1024),
    ("tp8_row_shard_down_k1792_n4096", 4096, 4096),
])
def test_gemm_tensor_parallel_shard_parity(name, Mmax, M):
    """One GPU's shard of an 8-way tensor-parallel layer (column shard of
    the QKV projection, row shard of the down-projection), every output
    element against the oracle's forward."""
    say(f"awq_gemm shard {name} M={M}")
    p = awq_inputs.workload_inputs(name, Mmax, 128)
    d = to_dev(p)
    y = run_gemm(d, M=M)
    del d
    ref = oracle.awq_linear_ref(p["x"][:M], p["qweight"], p["qzeros"], p["scales"], p["bias"], 128)
    assert ref.shape == y.shape
    assert_within_tol(y, ref, f"{name} M={M}")


# ------------------------------------------------- exact special cases
@pytest.mark.parametrize("name,Mmax,g,M", [
    ("decode_sweep_k8192_n7168", 16, 128, 16),
    ("decode_sweep_k8192_n7168", 16, 128, 1),   # one row: eight waves of two steps
    ("mlp_down_k14336_n4096", 4096, 128, 1),
    ("mlp_down_k14336_n4096", 4096, -1, 1),
    ("decode_sweep_k8192_n7168", 16, 128, 3),   # the atomic exchange, several rows
    ("decode_k8192_n1280", 1, 128, 1),
    ("mlp_down_k14336_n4096", 4096, -1, 3),
    ("prefill_qkv_m2048_k4096_n12288", 2048, 128, 256),
    ("mlp_down_k14336_n4096", 4096, 128, 256),
    ("midm_k8192_n7168", 128, 128, 32),   # decode, two row blocks
])
def test_one_hot_rows_exact(name, Mmax, g, M):
    """x rows one-hot at k_i, no bias: y[i] must equal the float16
    dequantised row k_i bit for bit (one exact product per output)."""
    say(f"one-hot {name} M={M} g={g}")
    p, w = cached_problem(name, Mmax, g)
    K = w.shape[0]
    ks = np.random.default_rng(99).choice(K, M, replace=M > K)
    ks[0], ks[-1] = 0, K - 1
    x = np.zeros((M, K), dtype=np.float16)
    x[np.arange(M), ks] = 1.0
    d = to_dev(dict(p, x=x, bias=None))
    y = run_gemm(d)
    np.testing.assert_array_equal(y.view(np.uint16), w[ks].view(np.uint16))


@pytest.mark.parametrize("M,K,N,g", [(1, 8192, 1280, 128), (1, 8192, 7168, 128),
                                     (1, 14336, 4096, -1), (16, 4096, 1024, 64),
                                     (5, 512, 40, 32), (300, 1024, 640, 128),
                                     (64, 512, 256, -1)])
def test_q_equal_z_gives_bias_exactly(M, K, N, g):
    """q == z everywhere: every kernel subtracts z per weight in exact float16
    integer arithmetic, so y is exactly the bias (exactly 0 without one)."""
    say(f"q==z M={M} K={K} N={N} g={g}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=M + K, bias=True, scale_lo=-1, scale_hi=1)
    gg = K if g == -1 else g
    p["qweight"] = np.repeat(p["qzeros"], gg, axis=0)
    d = to_dev(p)
    y = run_gemm(d)
    np.testing.assert_array_equal(y.view(np.uint16),
                                  np.broadcast_to(p["bias"], (M, N)).view(np.uint16))
    d["bias"] = None
    y0 = run_gemm(d)
    assert np.all(y0 == 0)


@pytest.mark.parametrize("M", [1, 16, 256])
def test_group_minus_one_bit_identical_to_K(M):
    say(f"g=-1 vs g=K M={M}")
    p = awq_inputs.make_inputs(M, 2048, 512, -1, seed=5)
    d = to_dev(p)
    a = run_gemm(d)
    d["group_size"] = 2048
    b = run_gemm(d)
    np.testing.assert_array_equal(a.view(np.uint16), b.view(np.uint16))


# ------------------------------------------- forced paths, tails, edges
@pytest.mark.parametrize("path,M,K,N,g,bias", [
    ("decode", 16, 4096, 12288, 128, True),
    ("decode", 3, 256, 40, 64, True),
    ("decode", 5, 96, 24, -1, False),
    ("decode", 2, 64, 8, 32, True),
    ("prefill", 1, 8192, 7168, 128, False),
    ("prefill", 16, 1024, 1280, 128, True),
    ("prefill", 17, 264, 136, 8, True),
    ("prefill", 255, 72, 24, 4, False),
    ("prefill", 257, 520, 392, 8, True),
    ("prefill", 31, 40, 40, -1, True),
    ("prefill", 300, 96, 200, 32, True),
    ("prefill", 513, 208, 264, 16, True),
    ("prefill", 64, 192, 128, 64, False),
    ("prefill", 2, 8, 8, -1, True),
    ("prefill", 300, 2000, 264, 16, True),    # split K: 4 splits, K tail, ragged M and N
    ("prefill", 64, 1536, 256, 128, False),   # split K: 3 splits
    ("prefill", 256, 2048, 512, 128, True),   # split K: 4 splits of whole tiles
    ("generic", 4, 256, 128, 64, True),
    ("generic", 33, 96, 24, 3, True),
    ("generic", 2, 100, 40, -1, False),
    ("generic", 17, 12, 8, 1, True),
])
def test_forced_path_and_tails(path, M, K, N, g, bias):
    say(f"forced {path} M={M} K={K} N={N} g={g}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=M * 7 + K + N, bias=bias)
    d = to_dev(p)
    y = run_gemm(d, path=path)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    assert_within_tol(y, ref, f"{path} M={M} K={K} N={N} g={g}")


# Decode with two 16-row MFMA blocks (17-32 rows): the streaming variant with
# one quantisation group per wave, split K summed by the second kernel.
@pytest.mark.parametrize("M,K,N,g,bias,opts", [
    (17, 8192, 7168, 128, True, None),                  # planner's choice: 4 steps, 16 splits
    (32, 8192, 7168, 128, False, None),
    (24, 14336, 4096, -1, True, None),                  # eight waves (14 splits), one group
    (32, 4096, 4096, 64, True, {"force_path": "decode"}),                   # 2 steps per wave
    (29, 2080, 96, 32, True, {"force_path": "decode"}),  # 1 step, K tail, one partial tile
    (31, 1024, 512, 128, True, {"force_path": "decode", "decode_steps": 4}),
    (18, 2048, 256, 128, True, {"force_path": "decode", "decode_waves": 8}),
    (32, 256, 64, -1, True, {"force_path": "decode"}),   # one split: no exchange
    (20, 4096, 2048, 64, False, {"force_path": "decode", "decode_steps": 4}),  # 4 would span
                                                                               # groups: 2 taken
])
def test_decode_two_row_blocks(M, K, N, g, bias, opts):
    say(f"decode two blocks M={M} K={K} N={N} g={g} opts={opts}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=M * 3 + K + N, bias=bias)
    d = to_dev(p)
    with awq.options(**(opts or {})):
        assert awq.gemm_plan(M, K, N, g)[0] == binding.AWQ_PATH_DECODE
    y = run_gemm(d, opts=opts)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    assert_within_tol(y, ref, f"decode two blocks M={M} K={K} N={N} g={g}")


# The split-K exchange the planner picks: the atomic exchange for at most
# four rows while a call issues fewer than 380K atomics, else two launches
# (also for M <= 4).  Each case against the oracle and 20 repeats bitwise.
@pytest.mark.parametrize("M,K,N,g,bias", [
    (3, 8192, 7168, 128, True),     # 344K atomics: atomic exchange
    (4, 8192, 7168, 128, False),    # 459K: two launches, eight waves
    (4, 4096, 4096, 128, True),     # 524K: two launches, four waves of one step
    (4, 4096, 12288, 64, False),    # two launches; g = 64: two steps, four waves
    (2, 14336, 4096, -1, True),     # 229K: atomic exchange, one group
])
def test_decode_exchange_choice(M, K, N, g, bias):
    say(f"decode exchange M={M} K={K} N={N} g={g}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=M + K + N + 7, bias=bias)
    d = to_dev(p)
    assert awq.gemm_plan(M, K, N, g)[0] == binding.AWQ_PATH_DECODE
    y = run_gemm(d)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    assert_within_tol(y, ref, f"decode exchange M={M} K={K} N={N} g={g}")
    first = awq.gemm(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g).clone()
    outs = [awq.gemm(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
            for _ in range(20)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), first.view(torch.int16))


WIDE = {"prefill_bn": 192}


@pytest.mark.parametrize("M,K,N,g,bias", [
    (300, 2000, 264, 16, True),    # K tail, ragged M, N = 192 + 72
    (513, 208, 392, 8, False),     # three row tiles, N = 2 * 192 + 8
    (256, 1024, 384, 128, True),   # whole tiles
    (64, 1536, 200, -1, True),     # one group, N = 192 + 8
    (1024, 4096, 768, 128, True),  # split K with the wide tile
])
def test_prefill_wide_tile(M, K, N, g, bias):
    """The 256 x 192 prefill tile, forced, on shapes that cut through its
    column blocks, row blocks and K steps."""
    say(f"wide prefill M={M} K={K} N={N} g={g}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=M + 3 * K + N, bias=bias)
    d = to_dev(p)
    y = run_gemm(d, path="prefill", opts=WIDE)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    assert_within_tol(y, ref, f"wide M={M} K={K} N={N} g={g}")


def test_prefill_wide_tile_exact_cases():
    """One-hot rows reproduce the dequantised rows bit for bit (positive
    scales: a weight of -0.0 would come out as +0.0, a sum that starts from
    zero) and q == z gives the bias bit for bit (scales of both signs)
    through the wide tile."""
    say("wide prefill exact cases")
    M, K, N, g = 300, 1024, 456, 64
    p = awq_inputs.make_inputs(M, K, N, g, seed=21, bias=True)
    w = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    ks = np.random.default_rng(5).choice(K, M)
    x = np.zeros((M, K), dtype=np.float16)
    x[np.arange(M), ks] = 1.0
    d = to_dev(dict(p, x=x, bias=None))
    y = run_gemm(d, path="prefill", opts=WIDE)
    np.testing.assert_array_equal(y.view(np.uint16), w[ks].view(np.uint16))
    p = awq_inputs.make_inputs(M, K, N, g, seed=22, bias=True, scale_lo=-1, scale_hi=1)
    p["qweight"] = np.repeat(p["qzeros"], g, axis=0)
    d = to_dev(p)
    y = run_gemm(d, path="prefill", opts=WIDE)
    np.testing.assert_array_equal(y.view(np.uint16),
                                  np.broadcast_to(p["bias"], (M, N)).view(np.uint16))


@pytest.mark.parametrize("bm,M,K,N,g,bias", [
    (64, 17, 4096, 1024, 128, True),    # split K, one row tile mostly padding
    (64, 64, 2000, 264, 16, False),     # K tail, N = 2 * 128 + 8
    (64, 200, 512, 384, 64, True),      # four row tiles, the last ragged
    (128, 65, 8192, 1280, 128, True),   # split K
    (128, 300, 1032, 136, -1, False),   # one group, K tail, N = 128 + 8
    (128, 128, 256, 512, 8, True),      # whole tiles, short K (no split)
])
def test_prefill_short_tiles(bm, M, K, N, g, bias):
    """The 64- and 128-row prefill tiles (forced), on shapes that cut through
    their row blocks, column blocks and K steps."""
    say(f"prefill BM={bm} M={M} K={K} N={N} g={g}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=bm + M + K + N, bias=bias)
    d = to_dev(p)
    y = run_gemm(d, path="prefill", opts={"prefill_bm": bm})
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    assert_within_tol(y, ref, f"BM={bm} M={M} K={K} N={N} g={g}")


@pytest.mark.parametrize("bm", [64, 128])
def test_prefill_short_tiles_exact(bm):
    """One-hot rows and q == z stay exact with the short tiles (split K
    included: the reduction adds exact zeros)."""
    say(f"prefill BM={bm} exact cases")
    M, K, N, g = bm - 3, 2048, 520, 64
    opts = {"prefill_bm": bm}
    p = awq_inputs.make_inputs(M, K, N, g, seed=bm)
    w = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    ks = np.random.default_rng(bm).choice(K, M)
    x = np.zeros((M, K), dtype=np.float16)
    x[np.arange(M), ks] = 1.0
    y = run_gemm(to_dev(dict(p, x=x, bias=None)), path="prefill", opts=opts)
    np.testing.assert_array_equal(y.view(np.uint16), w[ks].view(np.uint16))
    q = awq_inputs.make_inputs(M, K, N, g, seed=bm + 1, bias=True, scale_lo=-1, scale_hi=1)
    q["qweight"] = np.repeat(q["qzeros"], g, axis=0)
    y = run_gemm(to_dev(q), path="prefill", opts=opts)
    np.testing.assert_array_equal(y.view(np.uint16),
                                  np.broadcast_to(q["bias"], (M, N)).view(np.uint16))


@pytest.mark.parametrize("M", [2, 3, 17, 31, 255])
def test_mid_batch_tails(M):
    say(f"batch tail M={M}")
    p = awq_inputs.make_inputs(M, 4096, 1024, 128, seed=M, bias=True)
    d = to_dev(p)
    y = run_gemm(d)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], 128)
    assert_within_tol(y, ref, f"M={M}")


@pytest.mark.parametrize("M,K,N,g,bm,bn,bias", [
    (300, 1024, 768, 128, 256, 192, True),   # 16x16x32 wide tile, ragged rows
    (256, 2048, 520, 64, 256, 128, False),   # 16x16x32 narrow tile, ragged columns
    (260, 1000, 384, -1, 256, 192, True),    # 16x16x32, partial last K step
    (100, 1024, 256, 128, 128, 128, True),   # 32x32x16 tile
])
def test_prefill_unaligned_out_direct_stores(M, K, N, g, bm, bn, bias):
    """y only 2-byte aligned: with one split the prefill stores each element
    from its accumulators instead of staging the tile in LDS."""
    say(f"prefill unaligned out M={M} K={K} N={N} g={g} tile {bm}x{bn}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=M + N, bias=bias)
    d = to_dev(p)
    buf = torch.full((M * N + 1,), float("nan"), dtype=torch.float16, device=DEV)
    y = buf[1:].view(M, N)
    assert y.data_ptr() % 16 != 0
    with awq.options(force_path=binding.AWQ_PATH_PREFILL, prefill_bm=bm, prefill_bn=bn,
                     prefill_splits=1):
        assert awq.gemm_plan(M, K, N, g)[0] == binding.AWQ_PATH_PREFILL
        awq.gemm(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g, out=y)
        torch.cuda.synchronize()
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    assert_within_tol(y.cpu().numpy(), ref, f"unaligned out {bm}x{bn}")
    assert torch.isnan(buf[0]).item()   # nothing written before y


def test_unaligned_x_takes_general_kernel():
    say("unaligned x")
    p = awq_inputs.make_inputs(3, 512, 256, 128, seed=31, bias=True)
    d = to_dev(p)
    buf = torch.empty(3 * 512 + 1, dtype=torch.float16, device=DEV)
    x = buf[1:].view(3, 512)
    x.copy_(d["x"])
    assert x.data_ptr() % 16 != 0
    path, _ = awq.gemm_plan(3, 512, 256, 128, x.data_ptr(), d["scales"].data_ptr())
    assert path == binding.AWQ_PATH_GENERIC
    y = awq.gemm(x, d["qweight"], d["qzeros"], d["scales"], d["bias"], 128)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], 128)
    assert_within_tol(y.cpu().numpy(), ref, "unaligned x")


def test_empty_batch_and_leading_dims():
    say("empty batch, leading dims")
    p = awq_inputs.make_inputs(6, 256, 128, 64, seed=3, bias=True)
    d = to_dev(p)
    y0 = awq.gemm(d["x"][:0], d["qweight"], d["qzeros"], d["scales"], d["bias"], 64)
    assert y0.shape == (0, 128)
    y3 = awq.gemm(d["x"].view(2, 3, 256), d["qweight"], d["qzeros"], d["scales"], d["bias"], 64)
    assert y3.shape == (2, 3, 128)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], 64)
    assert_within_tol(y3.reshape(6, 128).cpu().numpy(), ref, "leading dims")


@pytest.mark.parametrize("M", [1, 16, 32, 256, 2048])
def test_deterministic_repeats(M):
    """Split-K partials are summed in a fixed order: repeats are bitwise equal."""
    say(f"determinism M={M}")
    p = awq_inputs.make_inputs(M, 4096, 2048, 128, seed=M, bias=True)
    d = to_dev(p)
    first = awq.gemm(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], 128).clone()
    outs = [awq.gemm(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], 128)
            for _ in range(100)]
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(y.view(torch.int16), first.view(torch.int16))


def test_workspace_reuse_across_shapes():
    """One workspace serves decode calls of different shapes (both exchange
    modes: M <= 4 atomic, M > 4 two-launch) and split-K prefill calls back
    to back: every call leaves the accumulator region zero."""
    say("workspace reuse")
    ws = torch.zeros(awq.gemm_workspace_size(16, 8192, 7168, 128), dtype=torch.uint8, device=DEV)
    shapes = [(16, 8192, 7168), (1, 8192, 1280), (256, 2048, 512), (4, 4096, 2048),
              (8, 4096, 1280), (64, 1536, 256), (2, 8192, 7168), (16, 8192, 7168)]
    assert all(awq.gemm_workspace_size(M, K, N, 128) <= ws.numel() for M, K, N in shapes)
    for (M, K, N) in shapes:
        p = awq_inputs.make_inputs(M, K, N, 128, seed=K + M)
        d = to_dev(p)
        y = awq.gemm(d["x"], d["qweight"], d["qzeros"], d["scales"], None, 128, workspace=ws)
        ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], None, 128)
        assert_within_tol(y.cpu().numpy(), ref, f"reuse M={M} K={K} N={N}")
        assert torch.count_nonzero(ws[:ZERO_REGION]).item() == 0, f"dirty after M={M} K={K} N={N}"


@pytest.mark.parametrize("lds", [True, False])
def test_decode_large_partials_take_float_path(lds):
    """A split's partial beyond the fixed-point range of the split-K exchange
    (|p| >= 2^21) is published as a float: one activation of 60000 in a group
    whose scales are 100 makes those outputs overflow to +-inf in float16,
    exactly as the oracle's do, while the columns it does not reach stay
    within tolerance.  The workspace is clean afterwards."""
    N = 1280 if lds else 1288
    K, g, k0 = 8192, 128, 5000
    say(f"decode float path N={N}")
    p = awq_inputs.make_inputs(2, K, N, g, seed=17, bias=True)
    p["x"][0, k0] = np.float16(60000.0)
    p["scales"][k0 // g, :] = np.float16(100.0)
    assert awq.gemm_plan(2, K, N, g)[0] == binding.AWQ_PATH_DECODE
    d = to_dev(p)
    ws = torch.zeros(awq.gemm_workspace_size(2, K, N, g), dtype=torch.uint8, device=DEV)
    y = awq.gemm(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g,
                 workspace=ws).cpu().numpy().astype(np.float64)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    with np.errstate(over="ignore"):
        ref16 = ref.astype(np.float16).astype(np.float64)
    big = np.isinf(ref16)
    assert big[0].sum() > N // 2          # the float path was taken for most columns
    assert np.array_equal(np.isinf(y), big)
    assert np.array_equal(y[big], ref16[big])
    assert_within_tol(y[~big], ref[~big], "finite outputs")
    assert torch.count_nonzero(ws[:ZERO_REGION]).item() == 0
    q = awq_inputs.make_inputs(2, K, N, g, seed=18)
    dq = to_dev(q)
    y2 = awq.gemm(dq["x"], dq["qweight"], dq["qzeros"], dq["scales"], None, g, workspace=ws)
    ref2 = oracle.awq_linear_ref(q["x"], q["qweight"], q["qzeros"], q["scales"], None, g)
    assert_within_tol(y2.cpu().numpy(), ref2, "after float-path call")


def test_wqlinear_module_forward():
    say("WQLinear forward")
    p = awq_inputs.make_inputs(8, 1024, 512, 128, seed=8, bias=True)
    d = to_dev(p)
    layer = awq.WQLinear(4, 128, d["qweight"], d["qzeros"], d["scales"], d["bias"])
    y = layer(d["x"].view(2, 4, 1024))
    assert y.shape == (2, 4, 512)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], 128)
    assert_within_tol(y.reshape(8, 512).cpu().numpy(), ref, "WQLinear")


# ------------------------------------------------ the unquantised baseline
@pytest.mark.parametrize("M,K,N,bias", [
    (1, 8192, 1280, False),    # the pages' single-token shapes
    (1, 8192, 7168, True),
    (4, 8192, 7168, False),
    (3, 1000, 200, True),      # K not a multiple of 512: partial last chunk
    (2, 8, 9, True),           # one chunk, N not a multiple of 8 rows
])
def test_dense_gemv_parity(M, K, N, bias):
    """awq_dense_gemv (F.linear, weight (N, K)) against the float64 oracle."""
    say(f"dense M={M} K={K} N={N}")
    rng = np.random.default_rng(M + K + N)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    b = (rng.standard_normal(N) * 0.1).astype(np.float16) if bias else None
    xd, wd = torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV)
    bd = torch.from_numpy(b).to(DEV) if bias else None
    y = awq.dense_gemv(xd, wd, bd)
    ref = oracle.dense_linear_ref(x, w, b)
    assert_within_tol(y.cpu().numpy(), ref, f"dense M={M} K={K} N={N}")
    y2 = awq.dense_gemv(xd, wd, bd)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))   # fixed summation order


def test_dense_gemv_exact_cases():
    """One-hot rows return the selected weight column exactly; an empty
    batch launches nothing."""
    say("dense exact cases")
    K, N = 4096, 3000
    w = (np.random.default_rng(1).standard_normal((N, K))).astype(np.float16)
    ks = [0, 1234, K - 1]
    x = np.zeros((3, K), dtype=np.float16)
    x[np.arange(3), ks] = 1.0
    y = awq.dense_gemv(torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV)).cpu().numpy()
    np.testing.assert_array_equal(y.view(np.uint16), w.T[ks].view(np.uint16))
    y0 = awq.dense_gemv(torch.zeros((0, K), dtype=torch.float16, device=DEV),
                        torch.from_numpy(w).to(DEV))
    assert y0.shape == (0, N)


@pytest.mark.parametrize("M,K,N,g,steps", [(1, 8192, 7168, 128, 2), (3, 8192, 1280, 128, 1),
                                           (4, 14336, 4096, -1, 4), (2, 4096, 2048, 32, 2),
                                           (5, 8192, 7168, 128, 4), (8, 4096, 1280, 64, 2),
                                           (16, 14336, 4096, 128, 4), (13, 8192, 768, -1, 1)])
def test_decode_eight_waves(M, K, N, g, steps):
    """The decode work-group of eight waves along K (decode_waves=8; the
    atomic exchange up to 4 rows, the two-launch exchange above) against the
    oracle, and one-hot rows exact."""
    say(f"decode eight waves M={M} K={K} N={N} g={g} steps={steps}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=M + K + N + steps, bias=True)
    d = to_dev(p)
    opts = {"decode_waves": 8, "decode_steps": steps}
    y = run_gemm(d, path="decode", opts=opts)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    assert_within_tol(y, ref, f"eight waves M={M} K={K} N={N}")
    w = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    ks = np.random.default_rng(M).choice(K, M, replace=False)
    x = np.zeros((M, K), dtype=np.float16)
    x[np.arange(M), ks] = 1.0
    y1 = run_gemm(to_dev(dict(p, x=x, bias=None)), path="decode", opts=opts)
    np.testing.assert_array_equal(y1.view(np.uint16), w[ks].view(np.uint16))
