"""Parity of the row-to-group map (g_idx) entry points against the CPU oracle.

Bar: awq_dequant_gidx and awq_gather_rows bit-exact; awq_gemm_gidx and
awq_gemm_sorted within |gpu - ref| <= 1e-2 + 1e-2*|ref| elementwise against
the float64 oracle (oracle.awq_linear_gidx_ref on the ORIGINAL weight and
map, never the rebuilt one); exact where the arithmetic is exact (one-hot
rows).  Maps come from the seeded generators in awq_inputs.
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
ZERO_REGION = 4 * 65536 * 16   # accumulator region of a workspace


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


def test_dequant_gidx_unaligned_scales():
    """Scales that are not 16-byte aligned send awq_dequant_gidx to the
    one-word-per-thread kernel: the same bits as the oracle, including
    rows whose map entry is out of range (+0)."""
    say("dequant_gidx unaligned scales")
    K, N, G = 96, 72, 5
    p = problem(1, K, N, G, seed=41)
    gi = awq_inputs.random_g_idx(K, G, seed=42)
    gi[7], gi[50] = G, -3
    buf = torch.zeros(G * N + 1, dtype=torch.float16)
    buf[1:] = torch.from_numpy(p["scales"]).reshape(-1)
    sc = buf.to(DEV)[1:].view(G, N)
    w = awq.dequant_gidx(dev(p["qweight"]), dev(p["qzeros"]), sc, dev(gi)).cpu().numpy()
    good = gi.copy()
    good[[7, 50]] = 0
    ref = oracle.dequant_gidx(p["qweight"], p["qzeros"], p["scales"], good)
    ref[[7, 50]] = 0
    np.testing.assert_array_equal(w.view(np.uint16), ref.view(np.uint16))


def test_dequant_gidx_streamed_output_sampled_rows():
    """awq_dequant_gidx with a W larger than the last-level cache (K = 8192,
    N = 14336; nontemporal-store form) under an activation-order map:
    each row depends only on its packed row and its mapped group, so
    sampled rows are checked bit for bit against the oracle on those rows."""
    K, N, G = 8192, 14336, 64
    say(f"dequant_gidx streamed K={K} N={N} G={G}")
    p = problem(1, K, N, G, seed=31)
    gi = awq_inputs.act_order_g_idx(K, K // G, seed=32)
    w = awq.dequant_gidx(dev(p["qweight"]), dev(p["qzeros"]), dev(p["scales"]), dev(gi))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(33).choice(K, size=512, replace=False))
    rows[0], rows[-1] = 0, K - 1
    got = w[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    ref = oracle.dequant_gidx(p["qweight"][rows], p["qzeros"], p["scales"], gi[rows])
    np.testing.assert_array_equal(got.view(np.uint16), ref.view(np.uint16))


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


# ------------------------------------------------------------- gather_rows
@pytest.mark.parametrize("K,N,rows", [(1000, 520, 1000), (1024, 512, 1536), (8192, 7168, 8192)])
def test_gather_rows_bit_exact(K, N, rows):
    """Any index vector, repeats and out-of-range entries (zero rows)
    included."""
    say(f"gather_rows K={K} N={N} rows={rows}")
    p = awq_inputs.make_inputs(1, K, N, -1, seed=K)
    rng = np.random.default_rng(K)
    idx = rng.integers(-3, K + 3, size=rows).astype(np.int32)
    out = awq.gather_rows(dev(p["qweight"]), dev(idx)).cpu().numpy()
    ok = (idx >= 0) & (idx < K)
    np.testing.assert_array_equal(out[ok], p["qweight"][idx[ok]])
    assert np.all(out[~ok] == 0)
    sc = p["scales"]
    out_s = awq.gather_rows(dev(sc), dev(np.array([0, 0], dtype=np.int32))).cpu().numpy()
    np.testing.assert_array_equal(out_s.view(np.uint16), sc[[0, 0]].view(np.uint16))


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


# ------------------------------------------------------- sorted weights
def act_problem(M, K, N, g, seed, bias=False):
    p = awq_inputs.make_inputs(M, K, N, g, seed=seed, bias=bias)
    p["g_idx"] = awq_inputs.act_order_g_idx(K, g, seed=seed + 7)
    return p


def map_problem(M, K, N, G, seed, bias=False):
    """An arbitrary map: unequal, possibly empty or one-row groups."""
    p = problem(M, K, N, G, seed=seed, bias=bias)
    p["g_idx"] = awq_inputs.random_g_idx(K, G, seed=seed + 11)
    return p


def run_sorted(p, workspace=None):
    w = awq.prepare_gidx(dev(p["qweight"]), dev(p["qzeros"]), dev(p["scales"]), p["g_idx"])
    y = awq.gemm_sorted(dev(p["x"]), w, dev(p["bias"]) if p["bias"] is not None else None,
                        workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy(), w


def ref_of(p):
    return oracle.awq_linear_gidx_ref(p["x"], p["qweight"], p["qzeros"], p["scales"],
                                      p["g_idx"], p["bias"])


@pytest.mark.parametrize("M,K,N,g,bias", [
    (1, 4096, 1024, 128, False), (4, 4096, 1024, 128, True), (16, 2048, 512, 64, False),
    (3, 1024, 520, 128, True),                       # register decode variant (N % 32 != 0)
    (64, 2048, 768, 128, False), (256, 1024, 1024, 128, True), (301, 1024, 520, 32, False),
    (66, 14336, 256, 128, True),                      # x rows staged two per work-group
    (40, 20480, 128, 128, False),                     # one row per work-group
    (2, 996, 64, 4, False),                           # 4-row groups: 32-row blocks, padded
    (5, 4800, 256, 96, True),                         # 96-row groups: three blocks each
])
def test_sorted_act_order_parity(M, K, N, g, bias):
    """Activation-order maps: prepare_gidx + gemm_sorted against the
    oracle's forward of the original weight under its map."""
    say(f"sorted act order M={M} K={K} N={N} g={g}")
    p = act_problem(M, K, N, g, seed=M * 3 + K, bias=bias)
    y, w = run_sorted(p)
    whole = g >= 32 and g & (g - 1) == 0
    assert w.block_rows == (g if whole else 32)
    blocks = (K // g) * -(-g // 32)
    assert w.rows == (K if whole else 32 * (blocks + blocks % 2))
    assert_within_tol(y, ref_of(p), f"sorted act order M={M}")


@pytest.mark.parametrize("M,K,N,G,bias", [
    (1, 8192, 1024, 64, False), (4, 4096, 512, 37, True), (16, 2048, 256, 200, False),
    (33, 1024, 520, 5, True), (256, 4096, 768, 100, False), (7, 300, 64, 1000, True),
])
def test_sorted_any_map_parity(M, K, N, G, bias):
    """Arbitrary maps (unequal, empty and one-row groups) run on the grouped
    kernels after the blocked rebuild, against the oracle."""
    say(f"sorted any map M={M} K={K} N={N} G={G}")
    p = map_problem(M, K, N, G, seed=M + K + G, bias=bias)
    y, w = run_sorted(p)
    assert w.block_rows == 32 and w.rows % 64 == 0 and w.rows >= K
    assert_within_tol(y, ref_of(p), f"sorted any map M={M} G={G}")


@pytest.mark.parametrize("M,K,N,G", [(2, 1024, 256, 8), (64, 2048, 512, 23)])
def test_wqlinear_gidx_module(M, K, N, G):
    """WQLinearGidx: the map is taken at construction, forward flattens
    leading dimensions and matches the oracle's forward under the map; the
    module's buffers are the rebuilt weight."""
    say(f"WQLinearGidx M={M} K={K} N={N} G={G}")
    p = map_problem(M, K, N, G, seed=M + G, bias=True)
    layer = awq.WQLinearGidx(4, dev(p["qweight"]), dev(p["qzeros"]), dev(p["scales"]),
                             torch.from_numpy(p["g_idx"]), dev(p["bias"]))
    assert (layer.in_features, layer.out_features, layer.num_groups) == (K, N, G)
    assert layer.qweight.shape[0] == layer.perm.shape[0] >= K
    y = layer(dev(p["x"]).reshape(2, M // 2, K))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (2, M // 2, N)
    assert_within_tol(y.reshape(M, N).cpu().numpy(), ref_of(p), "WQLinearGidx")


@pytest.mark.parametrize("steps", [1, 2, 4, 8])
@pytest.mark.parametrize("M", [1, 5])
def test_sorted_decode_every_step_count(steps, M):
    """The LDS decode kernel gathers x through perm itself for 1, 2 and 4
    steps per wave (the load order differs with the step count); 8 steps
    take the separate reorder.  Forced through the decode_steps option;
    whole groups and padded blocks."""
    for p in (act_problem(M, 8192, 1024, 128, seed=steps * 10 + M, bias=True),
              map_problem(M, 8192, 1024, 50, seed=steps * 10 + M, bias=True)):
        say(f"sorted decode steps={steps} M={M} G={p['scales'].shape[0]}")
        with awq.options(decode_steps=steps):
            y, _ = run_sorted(p)
        assert_within_tol(y, ref_of(p), f"sorted decode steps={steps}")


@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_sorted_fused_and_separate_reorder(M):
    """Both forms of the decode's x reorder (gathered inside the decode
    kernel, or a separate pass first), forced through the
    decode_gather_max_m option, match the oracle at every decode batch, for
    a whole-group and a padded layout."""
    for p in (act_problem(M, 8192, 1280, 128, seed=70 + M, bias=True),
              map_problem(M, 8192, 1280, 70, seed=70 + M, bias=True)):
        ref = ref_of(p)
        for limit in (16, 0):
            say(f"sorted decode M={M} G={p['scales'].shape[0]} gather limit {limit}")
            with awq.options(decode_gather_max_m=limit):
                y = run_sorted(p)[0]
            assert_within_tol(y, ref, f"sorted M={M} limit {limit}")


@pytest.mark.parametrize("M,K,N,g", [(8, 4096, 1024, 128), (256, 2048, 768, 64)])
def test_sorted_one_hot_rows_exact(M, K, N, g):
    """x[i] = e_{k_i} selects row k_i of the dequantised map weight bit for
    bit: after the rebuild the single nonzero product is the same float16
    weight (decode and prefill kernels); also for a padded layout."""
    for p in (act_problem(M, K, N, g, seed=11 + M), map_problem(M, K, N, 45, seed=11 + M)):
        say(f"sorted one-hot M={M} G={p['scales'].shape[0]}")
        ks = np.random.default_rng(M).choice(K, size=M, replace=False)
        x = np.zeros((M, K), dtype=np.float16)
        x[np.arange(M), ks] = 1.0
        p["x"] = x
        y, _ = run_sorted(p)
        w = oracle.dequant_gidx(p["qweight"], p["qzeros"], p["scales"], p["g_idx"])
        np.testing.assert_array_equal(y.view(np.uint16), w[ks].view(np.uint16))


@pytest.mark.parametrize("M,K,N,g,rows", [(1, 8192, 7168, 128, [0]),
                                          (16, 8192, 7168, 128, [0, 7, 15]),
                                          (2048, 4096, 12288, 128, [0, 1023, 2047])])
def test_sorted_full_size_sampled(M, K, N, g, rows):
    """The decode and prefill sizes in the launch configuration the
    benchmark times, checked on sampled rows (activation order)."""
    say(f"sorted full size M={M} K={K} N={N}")
    p = act_problem(M, K, N, g, seed=M + 1, bias=(M == 2048))
    y, _ = run_sorted(p)
    w = oracle.dequant_gidx(p["qweight"], p["qzeros"], p["scales"], p["g_idx"])
    ref = p["x"][rows].astype(np.float64) @ w.astype(np.float64)
    if p["bias"] is not None:
        ref = ref + p["bias"].astype(np.float64)
    assert_within_tol(y[rows], ref, f"sorted full size M={M}")


def test_sorted_shares_workspace_with_gemm():
    """The reordered x sits after the region that must stay zero, so one
    workspace serves sorted and plain calls (atomic and two-launch decode
    exchanges, split prefill) back to back."""
    say("sorted workspace sharing")
    shapes = [(1, 8192, 7168), (16, 8192, 7168), (256, 2048, 512), (2, 4096, 1024)]
    need = max(max(awq.sorted_workspace_size(M, K, N, 128),
                   awq.gemm_workspace_size(M, K, N, 128)) for M, K, N in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for M, K, N in shapes:
        p = act_problem(M, K, N, 128, seed=K + M)
        y, _ = run_sorted(p, workspace=ws)
        assert_within_tol(y, ref_of(p), f"sorted M={M} K={K} N={N}")
        assert torch.count_nonzero(ws[:ZERO_REGION]).item() == 0
        d = {k: dev(p[k]) for k in ("x", "qweight", "qzeros", "scales")}
        y2 = awq.gemm(d["x"], d["qweight"], d["qzeros"], d["scales"], None, 128, workspace=ws)
        ref2 = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], None, 128)
        assert_within_tol(y2.cpu().numpy(), ref2, f"plain M={M} K={K} N={N}")
        assert torch.count_nonzero(ws[:ZERO_REGION]).item() == 0


def test_sorted_empty_batch():
    say("sorted: empty batch")
    p = act_problem(1, 256, 64, 64, seed=2)
    w = awq.prepare_gidx(dev(p["qweight"]), dev(p["qzeros"]), dev(p["scales"]), p["g_idx"])
    y = awq.gemm_sorted(torch.empty((0, 256), dtype=torch.float16, device=DEV), w)
    assert tuple(y.shape) == (0, 64)
