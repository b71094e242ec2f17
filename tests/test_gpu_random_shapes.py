"""Seeded random shapes through every kernel family and the sorted-weight
route, each checked against the CPU oracle.

The shapes are drawn once from a fixed seed (the list below is the same on
every run), spanning batch sizes across the decode / prefill boundary,
K and N that are and are not multiples of the tile sizes, group sizes of
every supported kind (and ones only the general kernel takes), bias or
not.  Bar as elsewhere: awq_dequant bit-exact; forwards within
|gpu - ref| <= 1e-2 + 1e-2*|ref| of the float64 oracle.
"""
import sys

import numpy as np
import pytest

import awq_inputs
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_weight_quantized_awq_amd as awq  # noqa: E402

DEV = "cuda:0"


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 40, 64, 100, 128, 200, 256, 300]))
        kind = rng.integers(0, 4)
        if kind == 0:      # contiguous power-of-two groups, K a multiple of the group
            g = int(rng.choice([32, 64, 128]))
            K = g * int(rng.integers(1, 33))
        elif kind == 1:    # one group
            g = -1
            K = 8 * int(rng.integers(1, 400))
        elif kind == 2:    # small power-of-two groups (prefill or general)
            g = int(rng.choice([4, 8, 16]))
            K = g * int(rng.integers(1, 129))
        else:              # group sizes only the general kernel takes
            g = int(rng.choice([3, 12, 24, 40]))
            K = g * int(rng.integers(1, 65))
        N = 8 * int(rng.integers(1, 161))
        out.append((M, K, N, g, bool(rng.integers(0, 2))))
    return out


SHAPES = _shapes(40, 2024)


def _large_shapes(n, seed):
    """Larger K and N (several decode splits and prefill tiles, ragged
    edges), batch sizes on both sides of every kernel boundary."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([1, 4, 7, 16, 33, 64, 97, 128, 129, 255, 256, 511]))
        g = int(rng.choice([32, 64, 128, -1]))
        K = (g if g > 0 else 64) * int(rng.integers(8, 65))
        N = 8 * int(rng.integers(64, 1025))
        out.append((M, K, N, g, bool(rng.integers(0, 2))))
    return out


LARGE_SHAPES = _large_shapes(16, 77)


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


def _check(y, ref, what):
    err = np.abs(y.astype(np.float64) - ref)
    bad = err > 1e-2 + 1e-2 * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} outside tolerance, max err {err.max():.3e}"


@pytest.mark.parametrize("M,K,N,g,bias", SHAPES)
def test_random_shape_gemm_and_dequant(M, K, N, g, bias):
    path = awq.PATH_NAMES[awq.gemm_plan(M, K, N, g)[0]]
    say(f"random shape M={M} K={K} N={N} g={g} bias={bias} ({path})")
    p = awq_inputs.make_inputs(M, K, N, g, seed=M * 7 + K + N, bias=bias)
    t = {k: torch.from_numpy(v).to(DEV) for k, v in p.items() if isinstance(v, np.ndarray)}
    y = awq.gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t.get("bias"), g)
    w = awq.dequant(t["qweight"], t["qzeros"], t["scales"], g)
    torch.cuda.synchronize()
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    _check(y.cpu().numpy(), ref, f"gemm {path}")
    wref = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint16), wref.view(np.uint16))


@pytest.mark.parametrize("M,K,N,g,bias", LARGE_SHAPES)
def test_large_random_shape_gemm(M, K, N, g, bias):
    """Larger seeded shapes through the planner's choice, against the
    float64 oracle on a sample of rows (first, last, and seeded ones)."""
    path = awq.PATH_NAMES[awq.gemm_plan(M, K, N, g)[0]]
    say(f"large random shape M={M} K={K} N={N} g={g} bias={bias} ({path})")
    p = awq_inputs.make_inputs(M, K, N, g, seed=M + K + N, bias=bias)
    t = {k: torch.from_numpy(v).to(DEV) for k, v in p.items() if isinstance(v, np.ndarray)}
    y = awq.gemm(t["x"], t["qweight"], t["qzeros"], t["scales"], t.get("bias"), g)
    torch.cuda.synchronize()
    rows = sorted({0, M - 1} | set(np.random.default_rng(M).integers(0, M, size=6).tolist()))
    ref = oracle.awq_linear_ref(p["x"][rows], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    _check(y.cpu().numpy()[rows], ref, f"gemm {path}")


@pytest.mark.parametrize("M,K,N,g,bias", SHAPES[:20])
def test_random_shape_under_random_map(M, K, N, g, bias):
    """The same shapes with a random row-to-group map over G groups (G drawn
    near K / 64): rebuilt as a sorted grouped weight, against the oracle's
    forward of the original weight under the map."""
    rng = np.random.default_rng(K + N)
    G = max(1, int(rng.integers(max(1, K // 128), max(2, K // 32) + 1)))
    say(f"random map M={M} K={K} N={N} G={G} bias={bias}")
    p = awq_inputs.make_inputs(M, K, N, -1, seed=M + K * 3 + N, bias=bias)
    qz = rng.integers(0, 2 ** 32, size=(G, N // 8), dtype=np.uint32).view(np.int32)
    sc = rng.uniform(0.001, 0.01, size=(G, N)).astype(np.float16)
    gi = awq_inputs.random_g_idx(K, G, seed=G + M)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    w = awq.prepare_gidx(d(p["qweight"]), d(qz), d(sc), gi)
    y = awq.gemm_sorted(d(p["x"]), w, d(p["bias"]) if bias else None)
    torch.cuda.synchronize()
    ref = oracle.awq_linear_gidx_ref(p["x"], p["qweight"], qz, sc, gi, p["bias"])
    _check(y.cpu().numpy(), ref, f"sorted map rows={w.rows}")
