"""Parity of the row-to-group map (g_idx) entry points against the CPU oracle.

Bar: awq_dequant_gidx and awq_permute_rows bit-exact; awq_gemm_gidx and
awq_gemm_act_order within |gpu - ref| <= 1e-2 + 1e-2*|ref| elementwise
against the float64 oracle (oracle.awq_linear_gidx_ref on the ORIGINAL
weight and map, never the reordered one); exact where the arithmetic is
exact (one-hot rows).  Maps come from the seeded generators in awq_inputs.
"""
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
ZERO_REGION = 65536 + 4 * 65536 * 16   # ticket + accumulator regions of a workspace


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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def assert_within_tol(gpu, ref, what):
    gpu = gpu.astype(np.float64)
    err = np.abs(gpu - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                             f"{i}: gpu={gpu[i]!r} ref={ref[i]!r}; max err {err.max():.3e}")


def problem(M, K, N, G, seed, bias=False):
    """Seeded inputs with G scale/zero rows (the map chooses among them)."""
    p = awq_inputs.make_inputs(M, K, N, -1, seed=seed, bias=bias)
    rng = np.random.default_rng(seed + 1)
    p["qzeros"] = rng.integers(0, 2 ** 32, size=(G, N // 8), dtype=np.uint32).view(np.int32)
    p["scales"] = rng.uniform(0.001, 0.01, size=(G, N)).astype(np.float16)
    return p


# ------------------------------------------------------------ dequant_gidx
@pytest.mark.parametrize("K,N,G,kind", [(96, 24, 3, "random"), (256, 136, 7, "random"),
                                        (1024, 520, 8, "act"), (8192, 7168, 64, "act")])
def test_dequant_gidx_bit_exact(K, N, G, kind):
    say(f"dequant_gidx K={K} N={N} G={G} {kind}")
    p = problem(1, K, N, G, seed=K + G)
    gi = (awq_inputs.random_g_idx(K, G, seed=G) if kind == "random"
          else awq_inputs.act_order_g_idx(K, K // G, seed=G))
    w = awq.dequant_gidx(dev(p["qweight"]), dev(p["qzeros"]), dev(p["scales"]), dev(gi))
    ref = oracle.dequant_gidx(p["qweight"], p["qzeros"], p["scales"], gi)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint16), ref.view(np.uint16))


def test_dequant_gidx_out_of_range_entries_give_zero_rows():
    """An entry outside [0, G) reads zero point 0 and scale 0: that row is
    +0 (documented behaviour of the device-side map; the host cannot check
    it), and the other rows are unaffected."""
    say("dequant_gidx out-of-range entries")
    K, N, G = 64, 32, 4
    p = problem(1, K, N, G, seed=5)
    gi = awq_inputs.random_g_idx(K, G, seed=6)
    bad = {5: G, 9: -1, 40: 1 << 30}
    good = gi.copy()
    for k, v in bad.items():
        gi[k] = v
    w = awq.dequant_gidx(dev(p["qweight"]), dev(p["qzeros"]), dev(p["scales"]),
                         dev(gi)).cpu().numpy()
    ref = oracle.dequant_gidx(p["qweight"], p["qzeros"], p["scales"], good)
    rows = np.array(sorted(bad))
    assert np.all(w[rows].view(np.uint16) == 0)
    keep = np.setdiff1d(np.arange(K), rows)
    np.testing.assert_array_equal(w[keep].view(np.uint16), ref[keep].view(np.uint16))


# ------------------------------------------------------------ permute_rows
@pytest.mark.parametrize("K,N", [(1000, 520), (1024, 512), (8192, 7168)])
def test_permute_rows_bit_exact(K, N):
    say(f"permute_rows K={K} N={N}")
    p = awq_inputs.make_inputs(1, K, N, -1, seed=K)
    perm = np.random.default_rng(K).permutation(K).astype(np.int32)
    out = awq.permute_rows(dev(p["qweight"]), dev(perm)).cpu().numpy()
    np.testing.assert_array_equal(out, p["qweight"][perm])


def test_permute_rows_out_of_range_entry_writes_zeros():
    say("permute_rows out-of-range entry")
    K, N = 64, 64
    p = awq_inputs.make_inputs(1, K, N, -1, seed=3)
    perm = np.arange(K, dtype=np.int32)[::-1].copy()
    perm[7] = K
    out = awq.permute_rows(dev(p["qweight"]), dev(perm)).cpu().numpy()
    assert np.all(out[7] == 0)
    keep = np.setdiff1d(np.arange(K), [7])
    np.testing.assert_array_equal(out[keep], p["qweight"][perm[keep]])


# --------------------------------------------------------------- gemm_gidx
@pytest.mark.parametrize("M,K,N,G,bias", [(1, 256, 136, 5, False), (5, 512, 64, 9, True),
                                          (17, 300, 200, 4, True), (40, 1024, 256, 16, False)])
def test_gemm_gidx_any_map(M, K, N, G, bias):
    """Arbitrary maps (unequal, possibly empty groups) through the general
    kernel."""
    say(f"gemm_gidx M={M} K={K} N={N} G={G}")
    p = problem(M, K, N, G, seed=M + K, bias=bias)
    gi = awq_inputs.random_g_idx(K, G, seed=M)
    y = awq.gemm_gidx(dev(p["x"]), dev(p["qweight"]), dev(p["qzeros"]), dev(p["scales"]),
                      dev(gi), dev(p["bias"]) if bias else None)
    ref = oracle.awq_linear_gidx_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], gi,
                                     p["bias"])
    assert_within_tol(y.cpu().numpy(), ref, "gemm_gidx")


# --------------------------------------------------------------- act order
def act_problem(M, K, N, g, seed, bias=False):
    p = awq_inputs.make_inputs(M, K, N, g, seed=seed, bias=bias)
    p["g_idx"] = awq_inputs.act_order_g_idx(K, g, seed=seed + 7)
    return p


def run_act_order(p, M=None, workspace=None):
    K = p["qweight"].shape[0]
    G = p["scales"].shape[0]
    qs, perm, gs = awq.prepare_act_order(dev(p["qweight"]), p["g_idx"], G)
    assert gs == K // G
    x = p["x"] if M is None else p["x"][:M]
    d = dict(qzeros=dev(p["qzeros"]), scales=dev(p["scales"]),
             bias=dev(p["bias"]) if p["bias"] is not None else None)
    y = awq.gemm_act_order(dev(x), perm, qs, d["qzeros"], d["scales"], d["bias"], gs,
                           workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("M,K,N,g,bias", [
    (1, 4096, 1024, 128, False), (4, 4096, 1024, 128, True), (16, 2048, 512, 64, False),
    (3, 1024, 520, 128, True),                       # register decode variant (N % 32 != 0)
    (64, 2048, 768, 128, False), (256, 1024, 1024, 128, True), (301, 1024, 520, 32, False),
    (66, 14336, 256, 128, True),                      # x rows staged two per work-group
    (40, 20480, 128, 128, False),                     # one row per work-group
    (2, 996, 64, 4, False),                           # K % 8 != 0: general kernel, scalar gather
])
def test_act_order_parity(M, K, N, g, bias):
    """prepare_act_order + gemm_act_order against the oracle's forward of the
    original weight under its activation-order map."""
    path = binding.PATH_NAMES[awq.gemm_plan(M, K, N, g)[0]]
    say(f"act order M={M} K={K} N={N} g={g} ({path})")
    p = act_problem(M, K, N, g, seed=M * 3 + K, bias=bias)
    y = run_act_order(p)
    ref = oracle.awq_linear_gidx_ref(p["x"], p["qweight"], p["qzeros"], p["scales"],
                                     p["g_idx"], p["bias"])
    assert_within_tol(y, ref, f"act order M={M}")


@pytest.mark.parametrize("steps", [1, 2, 4, 8])
@pytest.mark.parametrize("M", [1, 5])
def test_act_order_decode_every_step_count(steps, M, monkeypatch):
    """The LDS decode kernel gathers x through perm itself for 1, 2 and 4
    steps per wave (the load order differs with the step count); 8 steps
    take the separate reorder.  Forced through AWQ_DECODE_STEPS."""
    say(f"act order decode steps={steps} M={M}")
    monkeypatch.setenv("AWQ_DECODE_STEPS", str(steps))
    p = act_problem(M, 8192, 1024, 128, seed=steps * 10 + M, bias=True)
    assert awq.gemm_plan(M, 8192, 1024, 128)[0] == binding.AWQ_PATH_DECODE
    y = run_act_order(p)
    ref = oracle.awq_linear_gidx_ref(p["x"], p["qweight"], p["qzeros"], p["scales"],
                                     p["g_idx"], p["bias"])
    assert_within_tol(y, ref, f"act order decode steps={steps}")


@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_act_order_fused_and_separate_reorder(M, monkeypatch):
    """Both forms of the decode's x reorder (gathered inside the decode
    kernel, or a separate pass first), forced through
    AWQ_DECODE_GATHER_MAX_M, match the oracle at every decode batch."""
    p = act_problem(M, 8192, 1280, 128, seed=70 + M, bias=True)
    ref = oracle.awq_linear_gidx_ref(p["x"], p["qweight"], p["qzeros"], p["scales"],
                                     p["g_idx"], p["bias"])
    for limit in ("16", "0"):
        say(f"act order decode M={M} gather limit {limit}")
        monkeypatch.setenv("AWQ_DECODE_GATHER_MAX_M", limit)
        assert_within_tol(run_act_order(p), ref, f"act order M={M} limit {limit}")


@pytest.mark.parametrize("M,K,N,g", [(8, 4096, 1024, 128), (256, 2048, 768, 64)])
def test_act_order_one_hot_rows_exact(M, K, N, g):
    """x[i] = e_{k_i} selects row k_i of the dequantised map weight bit for
    bit: after the reorder the single nonzero product is the same float16
    weight (decode and prefill kernels)."""
    say(f"act order one-hot M={M}")
    p = act_problem(M, K, N, g, seed=11 + M)
    ks = np.random.default_rng(M).choice(K, size=M, replace=False)
    x = np.zeros((M, K), dtype=np.float16)
    x[np.arange(M), ks] = 1.0
    p["x"] = x
    y = run_act_order(p)
    w = oracle.dequant_gidx(p["qweight"], p["qzeros"], p["scales"], p["g_idx"])
    np.testing.assert_array_equal(y.view(np.uint16), w[ks].view(np.uint16))


@pytest.mark.parametrize("M,K,N,g,rows", [(1, 8192, 7168, 128, [0]),
                                          (16, 8192, 7168, 128, [0, 7, 15]),
                                          (2048, 4096, 12288, 128, [0, 1023, 2047])])
def test_act_order_full_size_sampled(M, K, N, g, rows):
    """The decode and prefill sizes in the launch configuration the
    benchmark times, checked on sampled rows."""
    say(f"act order full size M={M} K={K} N={N}")
    p = act_problem(M, K, N, g, seed=M + 1, bias=(M == 2048))
    y = run_act_order(p)
    w = oracle.dequant_gidx(p["qweight"], p["qzeros"], p["scales"], p["g_idx"])
    ref = p["x"][rows].astype(np.float64) @ w.astype(np.float64)
    if p["bias"] is not None:
        ref = ref + p["bias"].astype(np.float64)
    assert_within_tol(y[rows], ref, f"act order full size M={M}")


def test_act_order_shares_workspace_with_gemm():
    """The reordered x sits after the regions that must stay zero, so one
    workspace serves act-order and plain calls (atomic and ticket decode
    exchanges, split prefill) back to back."""
    say("act order workspace sharing")
    shapes = [(1, 8192, 7168), (16, 8192, 7168), (256, 2048, 512), (2, 4096, 1024)]
    need = max(max(awq.act_order_workspace_size(M, K, N, 128),
                   awq.gemm_workspace_size(M, K, N, 128)) for M, K, N in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for M, K, N in shapes:
        p = act_problem(M, K, N, 128, seed=K + M)
        y = run_act_order(p, workspace=ws)
        ref = oracle.awq_linear_gidx_ref(p["x"], p["qweight"], p["qzeros"], p["scales"],
                                         p["g_idx"], None)
        assert_within_tol(y, ref, f"act order M={M} K={K} N={N}")
        assert torch.count_nonzero(ws[:ZERO_REGION]).item() == 0
        d = {k: dev(p[k]) for k in ("x", "qweight", "qzeros", "scales")}
        y2 = awq.gemm(d["x"], d["qweight"], d["qzeros"], d["scales"], None, 128, workspace=ws)
        ref2 = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], None, 128)
        assert_within_tol(y2.cpu().numpy(), ref2, f"plain M={M} K={K} N={N}")
        assert torch.count_nonzero(ws[:ZERO_REGION]).item() == 0


def test_act_order_rejects_unequal_groups_and_empty_batch():
    say("act order: unequal groups, empty batch")
    gi = awq_inputs.random_g_idx(256, 5, seed=1)
    q = dev(awq_inputs.make_inputs(1, 256, 64, -1, seed=1)["qweight"])
    with pytest.raises(ValueError):
        awq.prepare_act_order(q, gi, 5)
    p = act_problem(1, 256, 64, 64, seed=2)
    qs, perm, gs = awq.prepare_act_order(dev(p["qweight"]), p["g_idx"], 4)
    y = awq.gemm_act_order(torch.empty((0, 256), dtype=torch.float16, device=DEV), perm, qs,
                           dev(p["qzeros"]), dev(p["scales"]), None, gs)
    assert tuple(y.shape) == (0, 64)
