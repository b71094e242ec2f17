"""The packed-weight 256-row prefill tile (packed 4-bit words staged in LDS,
dequantised by the matrix-core waves), forced through the prefill_packed
option, against the oracle: ragged rows and columns, both tile widths, every
group kind it takes, and the exact cases (one-hot rows select dequantised
rows bit for bit; q == z gives the bias bit for bit)."""
import sys

import numpy as np
import pytest

import awq_inputs
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_weight_quantized_awq_amd as awq  # noqa: E402
from bit_weight_quantized_awq_amd import binding  # noqa: E402

DEV = "cuda:0"
ATOL = RTOL = 1e-2


def say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    awq.lib()
    yield


# (tile width, prefill_packed option): 256 columns with one wave along M (of
# four), two (of four) or two of eight waves (3),
# (each wave all rows of 64 columns) or two (128 rows of 128 columns), and
# 192 columns (two waves along M).
TILES = [(256, 1), (256, 2), (256, 3), (192, 1)]


def run(p, g, tile):
    bn, mode = tile
    d = {k: (torch.from_numpy(v).to(DEV) if isinstance(v, np.ndarray) else v)
         for k, v in p.items()}
    with awq.options(force_path="prefill", prefill_packed=mode, prefill_bn=bn):
        M, K = p["x"].shape
        N = p["qweight"].shape[1] * 8
        assert awq.gemm_plan(M, K, N, g)[0] == binding.AWQ_PATH_PREFILL
        y = awq.gemm(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], g)
        torch.cuda.synchronize()
    return y.cpu().numpy()


def check(y, ref, what):
    err = np.abs(y.astype(np.float64) - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} bad, max err {err.max():.3e}"


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M,K,N,g,bias", [
    (256, 256, 256, 64, True),       # one whole tile
    (300, 1024, 448, 128, True),     # ragged rows and columns
    (513, 2048, 1024, -1, False),    # three row tiles, one group
    (1024, 4096, 768, 64, True),     # 64-row groups, many K steps
    (2048, 512, 4096, 512, False),   # groups of eight K steps
])
def test_packed_tile_parity(tile, M, K, N, g, bias):
    say(f"packed prefill {tile} M={M} K={K} N={N} g={g}")
    bn = tile[0]
    p = awq_inputs.make_inputs(M, K, N, g, seed=M + K + N + bn, bias=bias)
    y = run(p, g, tile)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    check(y, ref, f"packed {tile} M={M} K={K} N={N} g={g}")


@pytest.mark.parametrize("tile", TILES)
def test_packed_tile_exact_cases(tile):
    M, K, N, g = 300, 1024, 448, 64
    bn = tile[0]
    say(f"packed prefill exact cases {tile}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=31 + bn, bias=True)
    w = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    ks = np.random.default_rng(bn).choice(K, M)
    ks[0], ks[-1] = 0, K - 1
    x = np.zeros((M, K), dtype=np.float16)
    x[np.arange(M), ks] = 1.0
    y = run(dict(p, x=x, bias=None), g, tile)
    np.testing.assert_array_equal(y.view(np.uint16), w[ks].view(np.uint16))
    q = awq_inputs.make_inputs(M, K, N, g, seed=32 + bn, bias=True, scale_lo=-1, scale_hi=1)
    q["qweight"] = np.repeat(q["qzeros"], g, axis=0)
    y = run(q, g, tile)
    np.testing.assert_array_equal(y.view(np.uint16),
                                  np.broadcast_to(q["bias"], (M, N)).view(np.uint16))


@pytest.mark.parametrize("name,Mmax,M,g", [
    ("prefill_qkv_m2048_k4096_n12288", 2048, 2048, 128),
    ("mlp_down_k14336_n4096", 4096, 4096, 128),
    ("mlp_down_k14336_n4096", 4096, 4096, -1),
])
def test_packed_tile_workloads(name, Mmax, M, g):
    """The full-size prefill workloads through the packed tile, every output
    against the oracle."""
    say(f"packed prefill workload {name} M={M} g={g}")
    p = awq_inputs.workload_inputs(name, Mmax, g)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    for tile in TILES:
        y = run(p, g, tile)
        check(y, ref, f"{name} {tile}")
