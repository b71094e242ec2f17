"""The forward captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI
calls) and replayed: every replay must equal an eager call on the same
inputs bit for bit (the kernels sum in a fixed order), with new inputs
copied into the captured buffers, eager work and synchronisations between
the replays.

The atomic split-K exchange leaves its workspace accumulators at zero on
exit, so a graph can be replayed without clearing anything in between; the workspace is
zeroed once, eagerly, before capture (nothing is cleared inside the graph).
awq_gemm_noalloc is called once eagerly first, so that its one-time scratch
fill runs outside the capture.
"""
import numpy as np
import pytest

import awq_inputs
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_weight_quantized_awq_amd as awq  # noqa: E402
from bit_weight_quantized_awq_amd import binding  # noqa: E402
from test_gpu_parity import ZERO_REGION, assert_within_tol, say, to_dev  # noqa: E402

DEV = "cuda:0"
REPLAYS = 5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    awq.lib()
    yield


def _replay_and_compare(fn_capture, fn_eager, x_static, y_static, M, K, seed):
    """Captures fn_capture() (writes y_static from x_static) on a side stream,
    then replays it REPLAYS times with fresh x; each replay is compared with
    fn_eager(x) bit for bit."""
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn_capture()                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        fn_capture()
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    for i in range(REPLAYS):
        xi = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float16)).to(DEV)
        x_static.copy_(xi)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = y_static.clone()
        ref = fn_eager(xi)                 # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {i} differs"
    return got, xi


@pytest.mark.parametrize("M,K,N,g,bias", [
    (1, 8192, 7168, 128, False),      # decode, atomic exchange
    (16, 4096, 2048, 64, True),       # decode, two-launch exchange
    (24, 8192, 7168, 128, True),      # decode, two row blocks, eight waves
    (4, 14336, 4096, -1, False),      # decode, one group
    (256, 14336, 4096, 128, False),   # prefill, split K + reduce kernel
    (512, 2048, 4096, 128, True),     # prefill, one split
])
def test_graph_replay_matches_eager(M, K, N, g, bias):
    say(f"graph replay M={M} K={K} N={N} g={g} bias={bias}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=M + N, bias=bias)
    d = to_dev(p)
    ws = torch.zeros(max(1, awq.gemm_workspace_size(M, K, N, g)), dtype=torch.uint8, device=DEV)
    ws_eager = torch.zeros_like(ws)
    x_static = d["x"].clone()
    y_static = torch.empty((M, N), dtype=torch.float16, device=DEV)

    def capture():
        awq.gemm(x_static, d["qweight"], d["qzeros"], d["scales"], d["bias"], g, out=y_static,
                 workspace=ws)

    def eager(x):
        return awq.gemm(x, d["qweight"], d["qzeros"], d["scales"], d["bias"], g,
                        workspace=ws_eager)

    got, x_last = _replay_and_compare(capture, eager, x_static, y_static, M, K, seed=K + M)
    ref = oracle.awq_linear_ref(x_last.cpu().numpy(), p["qweight"], p["qzeros"], p["scales"],
                                p["bias"], g)
    assert_within_tol(got.cpu().numpy(), ref, f"graph replay M={M}")
    if awq.gemm_plan(M, K, N, g)[0] == binding.AWQ_PATH_DECODE:
        # The exchange left its accumulators at zero for the next replay.
        assert torch.count_nonzero(ws[:min(ZERO_REGION, ws.numel())]).item() == 0


@pytest.mark.parametrize("M,K,N", [(4, 8192, 7168), (17, 8192, 7168), (64, 8192, 7168)])
def test_graph_replay_noalloc(M, K, N):
    say(f"graph replay noalloc M={M} K={K} N={N}")
    g = 128
    p = awq_inputs.make_inputs(M, K, N, g, seed=M + 3, bias=True)
    d = to_dev(p)
    x_static = d["x"].clone()
    y_static = torch.empty((M, N), dtype=torch.float16, device=DEV)
    awq.gemm_noalloc(x_static, d["qweight"], d["qzeros"], d["scales"], d["bias"], g, out=y_static)
    torch.cuda.synchronize()

    def capture():
        awq.gemm_noalloc(x_static, d["qweight"], d["qzeros"], d["scales"], d["bias"], g,
                         out=y_static)

    def eager(x):
        return awq.gemm(x, d["qweight"], d["qzeros"], d["scales"], d["bias"], g)

    _replay_and_compare(capture, eager, x_static, y_static, M, K, seed=M + 11)


def test_graph_replay_sorted_weight():
    """The sorted-weight forward (activation-ordered groups) under replay."""
    M, K, N, g = 2, 4096, 2048, 128
    say(f"graph replay sorted M={M} K={K} N={N}")
    p = awq_inputs.make_inputs(M, K, N, g, seed=21)
    d = to_dev(p)
    g_idx = awq_inputs.act_order_g_idx(K, g, seed=5)
    w = awq.prepare_gidx(d["qweight"], d["qzeros"], d["scales"], g_idx)
    ws = torch.zeros(max(1, awq.sorted_workspace_size(M, w.rows, N, w.block_rows)),
                     dtype=torch.uint8, device=DEV)
    ws_eager = torch.zeros_like(ws)
    x_static = d["x"].clone()
    y_static = torch.empty((M, N), dtype=torch.float16, device=DEV)

    def capture():
        awq.gemm_sorted(x_static, w, None, out=y_static, workspace=ws)

    def eager(x):
        return awq.gemm_sorted(x, w, None, workspace=ws_eager)

    got, x_last = _replay_and_compare(capture, eager, x_static, y_static, M, K, seed=8)
    ref = oracle.awq_linear_gidx_ref(x_last.cpu().numpy(), p["qweight"], p["qzeros"],
                                     p["scales"], g_idx, None)
    assert_within_tol(got.cpu().numpy(), ref, "graph replay sorted")
