"""The largest packed weight the library takes: K * N just under 2^31
elements (qweight 1 GiB, every 32-bit byte offset of the fast kernels near
its range), through the C ABI, on sampled columns against the oracle.

K = 32768 with N = 65504 (the LDS-streaming decode variant, N % 32 == 0:
8 steps per wave, 32 splits; 4 steps would give 64, one more than the
exchange counts) and K = 32000 with N = 65528 (the register variant, two
waves along K: 63 splits).  The prefill tiles run unsplit.  The oracle runs
on the column slice that holds the sampled columns: packed words are whole
groups of 8 columns, so
qweight[:, words], qzeros[:, words] and the matching scale and bias columns
are a problem of their own whose outputs are exactly those columns'.

Bar as elsewhere: |gpu - ref| <= 1e-2 + 1e-2*|ref|; awq_dequant bit-exact.
"""
import functools

import numpy as np
import pytest

import awq_inputs
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_weight_quantized_awq_amd as awq  # noqa: E402
from bit_weight_quantized_awq_amd import binding  # noqa: E402
from test_gpu_parity import assert_within_tol, say  # noqa: E402

DEV = "cuda:0"
G = 128
M_MAX = 200
SHAPES = [(32768, 65504), (32000, 65528)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    awq.lib()
    yield
    _problem.cache_clear()
    torch.cuda.empty_cache()


@functools.lru_cache(maxsize=2)
def _problem(K, N):
    assert K * N < 2 ** 31
    p = awq_inputs.make_inputs(M_MAX, K, N, G, seed=N % 1000, bias=True)
    d = {k: torch.from_numpy(v).to(DEV) for k, v in p.items() if isinstance(v, np.ndarray)}
    return p, d


def _slice(p, words, M):
    """The sub-problem of the columns held by packed words `words`."""
    cols = (8 * words[:, None] + np.arange(8)[None, :]).ravel()
    return cols, dict(x=p["x"][:M], qweight=np.ascontiguousarray(p["qweight"][:, words]),
                      qzeros=np.ascontiguousarray(p["qzeros"][:, words]),
                      scales=np.ascontiguousarray(p["scales"][:, cols]),
                      bias=p["bias"][cols])


def _words(N, seed):
    nw = N // 8
    rng = np.random.default_rng(seed)
    # The first and last words (the ends of every row) and a random dozen.
    return np.unique(np.concatenate([[0, nw - 1], rng.choice(nw, 12, replace=False)]))


@pytest.mark.parametrize("M", [1, 16, M_MAX])
@pytest.mark.parametrize("K,N", SHAPES)
def test_largest_weight_forward(K, N, M):
    say(f"largest weight forward M={M} K={K} N={N}")
    p, d = _problem(K, N)
    path, _ = awq.gemm_plan(M, K, N, G)
    # M = 200 is past the decode kernel's 32 rows.
    assert path == (binding.AWQ_PATH_DECODE if M <= 32 else binding.AWQ_PATH_PREFILL)
    y = awq.gemm(d["x"][:M], d["qweight"], d["qzeros"], d["scales"], d["bias"], G)
    torch.cuda.synchronize()
    words = _words(N, M)
    cols, sub = _slice(p, words, M)
    ref = oracle.awq_linear_ref(sub["x"], sub["qweight"], sub["qzeros"], sub["scales"],
                                sub["bias"], G)
    got = y[:, torch.from_numpy(cols).to(DEV)].cpu().numpy()
    assert_within_tol(got, ref, f"largest weight M={M} N={N}")


@pytest.mark.parametrize("K,N", SHAPES)
def test_largest_weight_dequant(K, N):
    say(f"largest weight dequant K={K} N={N}")
    p, d = _problem(K, N)
    w = awq.dequant(d["qweight"], d["qzeros"], d["scales"], G)
    torch.cuda.synchronize()
    words = _words(N, 7)
    cols, sub = _slice(p, words, 1)
    ref = oracle.dequant(sub["qweight"], sub["qzeros"], sub["scales"], G)
    got = w[:, torch.from_numpy(cols).to(DEV)].cpu().numpy()
    np.testing.assert_array_equal(got.view(np.uint16), ref.view(np.uint16))
    del w
    torch.cuda.empty_cache()
