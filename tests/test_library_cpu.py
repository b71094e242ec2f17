"""Host-side tests of the C-ABI library: it loads without a GPU, exports every
symbol include/awq.h declares, and rejects every invalid argument before any
HIP call.  No compute runs here (no GPU in this environment)."""
import ctypes
import os
import re
import shutil
import subprocess
import sys

import pytest

import bit_weight_quantized_awq_amd as awq
from bit_weight_quantized_awq_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")

# Fake device addresses: never dereferenced, every call below returns before
# any HIP call.
A = 0x10000


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert header_functions() == sorted(binding.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = awq.lib()
    for name in header_functions():
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", binding.LIB_PATH],
                             capture_output=True, text=True, check=True).stdout
        exported = set(re.findall(r"\b(awq_\w+)\b", out))
        assert set(header_functions()) <= exported


def test_abi_version_matches_header():
    m = re.search(r"#define AWQ_ABI_VERSION (\d+)", open(HEADER).read())
    assert awq.abi_version() == int(m.group(1))


def test_status_strings():
    for s in range(6):
        assert awq.status_string(s)
    assert awq.status_string(0) == "success"
    assert awq.status_string(99) == "unknown status"


def _gemm(x=A, qw=A, qz=A, sc=A, bias=None, y=A, M=4, K=256, N=128, g=64, ws=None, wsb=0):
    return awq.lib().awq_gemm(x, qw, qz, sc, bias, y, M, K, N, g, ws, wsb, None)


def _dequant(qw=A, qz=A, sc=A, w=A, K=256, N=128, g=64):
    return awq.lib().awq_dequant(qw, qz, sc, w, K, N, g, None)


def _dense(x=A, w=A, bias=None, y=A, M=1, K=8192, N=1280):
    return awq.lib().awq_dense_gemv(x, w, bias, y, M, K, N, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(w=None), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(x=None), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(M=-1), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(K=0), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(N=0), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(M=5), binding.AWQ_ERROR_SHAPE),            # at most 4 rows
    (dict(K=100), binding.AWQ_ERROR_SHAPE),          # K % 8 != 0
    (dict(M=4, K=16392), binding.AWQ_ERROR_SHAPE),   # x does not fit the LDS stage
    (dict(x=A + 8), binding.AWQ_ERROR_MISALIGNED),
    (dict(w=A + 4), binding.AWQ_ERROR_MISALIGNED),
    (dict(y=A + 1), binding.AWQ_ERROR_MISALIGNED),
    (dict(bias=A + 1), binding.AWQ_ERROR_MISALIGNED),
    (dict(M=0, x=None, y=None), binding.AWQ_SUCCESS),  # empty batch: no launch
])
def test_dense_validation(kwargs, status):
    """The unquantised baseline rejects every invalid argument on the host."""
    assert _dense(**kwargs) == status


@pytest.mark.parametrize("kwargs,status", [
    (dict(qw=None), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(qz=None), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(sc=None), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(x=None), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(y=None), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(M=-1), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(K=0), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(N=0), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(N=-8), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(g=0), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(g=-2), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(N=100), binding.AWQ_ERROR_SHAPE),           # out_features % 8
    (dict(g=96), binding.AWQ_ERROR_SHAPE),            # in_features % group_size
    (dict(g=512), binding.AWQ_ERROR_SHAPE),           # group larger than K
    (dict(K=65536, N=65536, g=128), binding.AWQ_ERROR_SHAPE),  # K*N >= 2^31
    (dict(M=1 << 20, K=4096, N=4096), binding.AWQ_ERROR_SHAPE),  # M*K >= 2^31
    (dict(qw=A + 2), binding.AWQ_ERROR_MISALIGNED),
    (dict(qz=A + 1), binding.AWQ_ERROR_MISALIGNED),
    (dict(sc=A + 1), binding.AWQ_ERROR_MISALIGNED),
    (dict(x=A + 1), binding.AWQ_ERROR_MISALIGNED),
    (dict(y=A + 3), binding.AWQ_ERROR_MISALIGNED),
    (dict(bias=A + 1), binding.AWQ_ERROR_MISALIGNED),
    (dict(M=0, x=None, y=None), binding.AWQ_SUCCESS),  # empty batch: no launch
])
def test_gemm_validation(kwargs, status):
    assert _gemm(**kwargs) == status


def test_gemm_workspace_checked_before_launch():
    M, K, N, g = 1, 8192, 7168, 128
    need = awq.gemm_workspace_size(M, K, N, g)
    assert need > 0
    assert _gemm(M=M, K=K, N=N, g=g) == binding.AWQ_ERROR_WORKSPACE
    assert _gemm(M=M, K=K, N=N, g=g, ws=A, wsb=need - 1) == binding.AWQ_ERROR_WORKSPACE
    assert _gemm(M=M, K=K, N=N, g=g, ws=A + 8, wsb=need) == binding.AWQ_ERROR_MISALIGNED


@pytest.mark.parametrize("kwargs,status", [
    (dict(qw=None), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(w=None), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(K=0), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(N=12), binding.AWQ_ERROR_SHAPE),
    (dict(g=100), binding.AWQ_ERROR_SHAPE),
    (dict(g=-5), binding.AWQ_ERROR_INVALID_VALUE),
    (dict(w=A + 1), binding.AWQ_ERROR_MISALIGNED),
    (dict(qz=A + 2), binding.AWQ_ERROR_MISALIGNED),
])
def test_dequant_validation(kwargs, status):
    assert _dequant(**kwargs) == status


@pytest.mark.parametrize("M,K,N,g,path", [
    (4, 256, 128, 64, binding.AWQ_PATH_DECODE),
    (1, 8192, 1280, 128, binding.AWQ_PATH_DECODE),
    (16, 8192, 7168, 128, binding.AWQ_PATH_DECODE),
    (2048, 4096, 12288, 128, binding.AWQ_PATH_PREFILL),
    (1, 14336, 4096, -1, binding.AWQ_PATH_DECODE),
    (4096, 14336, 4096, -1, binding.AWQ_PATH_PREFILL),
    (256, 14336, 4096, 128, binding.AWQ_PATH_PREFILL),
    (17, 4096, 4096, 128, binding.AWQ_PATH_PREFILL),
    (4, 96, 64, 3, binding.AWQ_PATH_GENERIC),        # group size not a multiple of 4
    (4, 100, 64, -1, binding.AWQ_PATH_GENERIC),      # K % 8 != 0
    (4, 256, 64, 16, binding.AWQ_PATH_PREFILL),      # small groups: not decode
    (64, 384, 64, 96, binding.AWQ_PATH_GENERIC),     # group size not a power of two
    (64, 96, 64, -1, binding.AWQ_PATH_PREFILL),      # one group of any size
])
def test_plan_selects_kernel(M, K, N, g, path):
    got, ws = awq.gemm_plan(M, K, N, g)
    assert got == path
    if path == binding.AWQ_PATH_GENERIC:
        assert ws == 0
    else:
        assert ws <= awq.gemm_workspace_size(M, K, N, g)


def _prefill_splits_expected(M, K, N):
    """Split-K rule of the prefill kernel, restated: tiles of 64, 128 or 256
    rows (the smallest covering M, up to 256) by 128 columns; when there are
    fewer tiles than 256 CUs, up to 8 splits (no more than fill the CUs),
    each of at least 8 K steps of 64, none empty.  (Shapes that take the
    256 x 192 tile have enough tiles not to split.)"""
    bm = 64 if M <= 64 else (128 if M <= 128 else 256)
    tiles = -(-M // bm) * -(-N // 128)
    nkt = -(-K // 64)
    s = 1
    if tiles < 256:
        s = min(8, 256 // tiles, nkt // 8)
        s = s if s >= 2 else 1
    kps = -(-nkt // s)
    return -(-nkt // kps)


@pytest.mark.parametrize("M,K,N,g,splits", [
    (256, 14336, 4096, 128, 8),
    (1024, 14336, 4096, 128, 2),
    (2048, 4096, 12288, 128, 1),
    (4096, 14336, 4096, -1, 1),
    (300, 2000, 264, 16, 4),
    (17, 256, 4096, 128, 1),
    (64, 1536, 256, 128, 3),
    (17, 8192, 7168, 128, 4),     # 64-row tiles: 56 tiles
    (100, 4096, 1024, 128, 8),    # 128-row tiles: 8 tiles
])
def test_prefill_split_k_plan(M, K, N, g, splits):
    """Workspace of a split prefill, laid out like the decode exchange's: the
    4 MiB accumulator region, then one fp32 partial per split per output
    element; none without a split."""
    assert _prefill_splits_expected(M, K, N) == splits
    with awq.options(force_path="prefill"):
        path, ws = awq.gemm_plan(M, K, N, g)
    assert path == binding.AWQ_PATH_PREFILL
    assert ws == (0 if splits == 1 else 4 * 65536 * 16 + splits * M * N * 4)
    # The workspace size covers every kernel family that can run the problem:
    # up to 32 rows the decode kernel's too.
    if M > 32:
        assert awq.gemm_workspace_size(M, K, N, g) == ws
    else:
        assert awq.gemm_workspace_size(M, K, N, g) >= ws


def test_plan_unaligned_x_falls_back_to_generic():
    assert awq.gemm_plan(1, 8192, 7168, 128, x_ptr=A + 2, scales_ptr=A)[0] == \
        binding.AWQ_PATH_GENERIC
    assert awq.gemm_plan(1, 8192, 7168, 128, x_ptr=A, scales_ptr=A + 2)[0] == \
        binding.AWQ_PATH_GENERIC


def test_plan_size_limits():
    """The fast kernels address operands with 32-bit byte offsets: x and y up
    to 2^29 elements (1 GiB) take them; beyond, the general kernel (int
    element indices, valid while every operand stays below 2^31 elements).
    The largest packed weight (K * N just under 2^31) plans as decode with 8
    steps per wave, 32 splits."""
    assert awq.gemm_plan(1, 32768, 65504, 128)[0] == binding.AWQ_PATH_DECODE
    assert awq.gemm_plan(200, 32768, 65504, 128)[0] == binding.AWQ_PATH_PREFILL
    path, ws = awq.gemm_plan(1, 32768, 65504, 128)
    assert ws == 4 * 65536 * 16 + 32 * 1 * 65504 * 4
    assert awq.gemm_plan(16384, 32768, 64, 128)[0] == binding.AWQ_PATH_PREFILL   # x = 1 GiB
    assert awq.gemm_plan(16385, 32768, 64, 128)[0] == binding.AWQ_PATH_GENERIC
    assert awq.gemm_plan(8192, 64, 65536, -1)[0] == binding.AWQ_PATH_PREFILL     # y = 1 GiB
    assert awq.gemm_plan(8193, 64, 65536, -1)[0] == binding.AWQ_PATH_GENERIC
    # The register decode variant (N % 32 != 0) has two waves along K: up to
    # 63 splits of 8 steps, K <= 32256.
    assert awq.gemm_plan(16, 32000, 65528, 128)[0] == binding.AWQ_PATH_DECODE
    assert awq.gemm_plan(16, 32768, 65528, 128)[0] == binding.AWQ_PATH_PREFILL
    with pytest.raises(awq.AwqError):
        awq.gemm_plan(1, 65536, 32768, 128)                  # K * N = 2^31


def test_forced_path():
    with awq.options(force_path="prefill"):
        assert awq.gemm_plan(1, 8192, 7168, 128)[0] == binding.AWQ_PATH_PREFILL
        assert awq.get_option("force_path") == binding.AWQ_PATH_PREFILL
    assert awq.get_option("force_path") == binding.AWQ_OPT_AUTO
    assert awq.gemm_plan(1, 8192, 7168, 128)[0] == binding.AWQ_PATH_DECODE
    with awq.options(force_path="generic"):
        assert awq.gemm_plan(2048, 4096, 12288, 128)[0] == binding.AWQ_PATH_GENERIC
    with awq.options(force_path="decode"):
        with pytest.raises(awq.AwqError):
            awq.gemm_plan(64, 4096, 4096, 128)          # decode handles M <= 32 only


def test_option_values_checked():
    lib = binding.lib()
    for opt, bad in [(binding.AWQ_OPT_FORCE_PATH, 4), (binding.AWQ_OPT_FORCE_PATH, 0),
                     (binding.AWQ_OPT_DECODE_STEPS, 3), (binding.AWQ_OPT_DECODE_GATHER_MAX_M, 17),
                     (binding.AWQ_OPT_PREFILL_BM, 96), (binding.AWQ_OPT_PREFILL_BN, 64),
                     (binding.AWQ_OPT_PREFILL_SPLITS, 9), (binding.AWQ_OPT_DECODE_WAVES, 6), (binding.AWQ_OPT_PREFILL_PACKED, 4), (0, 1), (9, 1)]:
        assert lib.awq_set_option(opt, bad) == binding.AWQ_ERROR_INVALID_VALUE, (opt, bad)
    assert lib.awq_get_option(9, None) == binding.AWQ_ERROR_INVALID_VALUE
    assert lib.awq_get_option(binding.AWQ_OPT_PREFILL_BM, None) == binding.AWQ_ERROR_INVALID_VALUE
    with awq.options(prefill_bm=64, prefill_splits=3):
        assert awq.get_option("prefill_bm") == 64
        assert awq.get_option("prefill_splits") == 3
    assert awq.get_option("prefill_bm") == binding.AWQ_OPT_AUTO


def _plan_in_subprocess(env_extra, code):
    import subprocess
    env = dict(os.environ)
    for k in list(env):
        if k.startswith("AWQ_"):
            del env[k]
    env.update(env_extra)
    prog = ("import sys; sys.path.insert(0, %r)\n"
            "import bit_weight_quantized_awq_amd as awq\n"
            "from bit_weight_quantized_awq_amd import binding\n" % ROOT) + code
    res = subprocess.run([sys.executable, "-c", prog], env=env, capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    return res.stdout


def test_environment_read_once():
    """The AWQ_* variables seed the overrides on first use; changing the
    environment afterwards changes nothing."""
    out = _plan_in_subprocess({"AWQ_FORCE_PATH": "prefill", "AWQ_PREFILL_BM": "128"}, (
        "import os\n"
        "assert awq.gemm_plan(1, 8192, 7168, 128)[0] == binding.AWQ_PATH_PREFILL\n"
        "assert awq.get_option('prefill_bm') == 128\n"
        "os.environ['AWQ_FORCE_PATH'] = 'generic'\n"
        "assert awq.gemm_plan(1, 8192, 7168, 128)[0] == binding.AWQ_PATH_PREFILL\n"
        "awq.set_option('force_path', None)\n"
        "assert awq.gemm_plan(1, 8192, 7168, 128)[0] == binding.AWQ_PATH_DECODE\n"
        "print('ok')\n"))
    assert out.strip() == "ok"


def test_unrecognised_forced_path_fails_every_plan():
    out = _plan_in_subprocess({"AWQ_FORCE_PATH": "bogus"}, (
        "import ctypes\n"
        "try:\n"
        "    awq.gemm_plan(1, 4096, 4096, 128)\n"
        "    raise SystemExit('no error')\n"
        "except awq.AwqError as e:\n"
        "    assert e.status == binding.AWQ_ERROR_INVALID_VALUE\n"
        "lib = binding.lib()\n"
        "A = 0x10000\n"
        "st = lib.awq_gemm(A, A, A, A, None, A, 1, 4096, 4096, 128, None, 0, None)\n"
        "assert st == binding.AWQ_ERROR_INVALID_VALUE, st\n"
        "awq.set_option('force_path', None)\n"
        "assert awq.gemm_plan(1, 4096, 4096, 128)[0] == binding.AWQ_PATH_DECODE\n"
        "print('ok')\n"))
    assert out.strip() == "ok"


def test_decode_workspace_size_formula():
    """A fixed 4 MiB accumulator region (an 8-byte accumulator and an 8-byte
    mask per element, for M <= 4 and N <= 65536), then one fp32 slot per
    split per element; at most 63 splits."""
    for (M, K, N, g) in [(4, 8192, 7168, 128), (1, 14336, 4096, 128), (16, 8192, 1280, -1)]:
        path, ws = awq.gemm_plan(M, K, N, g)
        assert path == binding.AWQ_PATH_DECODE
        assert ws == awq.gemm_workspace_size(M, K, N, g)
        partial = ws - 4 * 65536 * 16
        assert partial % (M * N * 4) == 0
        splits = partial // (M * N * 4)
        assert 2 <= splits <= 63
        assert any(splits == -(-K // (128 * steps)) for steps in (1, 2, 4, 8))


@pytest.mark.parametrize("M,K,N,g,splits", [
    (1, 8192, 7168, 128, 16),   # 4 steps keep a wave in one 128-row group, 448 work-groups
    (16, 8192, 7168, 32, 16),   # no step count >= 2 keeps 32-row groups whole: largest with
    (1, 14336, 4096, 32, 28),   # enough work-groups (4 steps), not the most splits
    (1, 8192, 1280, 128, 32),   # too few work-groups anywhere: the most (2 steps)
])
def test_decode_step_choice(M, K, N, g, splits):
    """Decode step counts: the largest that keeps each wave in one group and
    gives enough work-groups; else the largest that gives enough; else the
    one with the most work-groups (fewer splits, less to exchange)."""
    path, ws = awq.gemm_plan(M, K, N, g)
    assert path == binding.AWQ_PATH_DECODE
    assert (ws - 4 * 65536 * 16) // (M * N * 4) == splits


def test_decode_split_limit():
    """K beyond 63 splits of 8 steps cannot take the decode kernel."""
    assert awq.gemm_plan(1, 63 * 1024, 4096, 128)[0] == binding.AWQ_PATH_DECODE
    assert awq.gemm_plan(1, 64 * 1024, 4096, 128)[0] != binding.AWQ_PATH_DECODE


def test_no_cpu_fallback():
    torch = pytest.importorskip("torch")
    q = torch.zeros((256, 16), dtype=torch.int32)
    with pytest.raises(ValueError, match="HIP device"):
        awq.gemm(torch.zeros((1, 256), dtype=torch.float16), q, torch.zeros((4, 16), dtype=torch.int32),
                 torch.zeros((4, 128), dtype=torch.float16), None, 64)
    with pytest.raises(ValueError, match="HIP device"):
        awq.dequant(q, torch.zeros((4, 16), dtype=torch.int32),
                    torch.zeros((4, 128), dtype=torch.float16), 64)


def test_wqlinear_construction_checks():
    torch = pytest.importorskip("torch")
    q = torch.zeros((256, 16), dtype=torch.int32)
    z = torch.zeros((4, 16), dtype=torch.int32)
    s = torch.zeros((4, 128), dtype=torch.float16)
    layer = awq.WQLinear(4, 64, q, z, s, None)
    assert layer.in_features == 256 and layer.out_features == 128
    assert layer.weight is layer.qweight
    assert awq.WQLinear(4, -1, q, z[:1], s[:1], None).group_size == 256
    with pytest.raises(ValueError):
        awq.WQLinear(8, 64, q, z, s, None)
    with pytest.raises(ValueError):
        awq.WQLinear(4, 100, q, z, s, None)


def test_wqlinear_gidx_construction_checks():
    """WQLinearGidx rejects other bit widths and, with no CPU fallback,
    tensors that are not on a HIP device (before any device work)."""
    torch = pytest.importorskip("torch")
    q = torch.zeros((64, 4), dtype=torch.int32)
    z = torch.zeros((2, 4), dtype=torch.int32)
    s = torch.zeros((2, 32), dtype=torch.float16)
    with pytest.raises(ValueError, match="4-bit"):
        awq.WQLinearGidx(8, q, z, s, [0] * 64, None)
    with pytest.raises(ValueError, match="HIP device"):
        awq.WQLinearGidx(4, q, z, s, [0] * 64, None)


def test_validation_under_sanitizers(tmp_path):
    """The HIP-free planning/validation translation unit, built with the host
    compiler under AddressSanitizer + UBSan and driven over a grid of
    arguments (including every error path and extreme sizes)."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    csrc = os.path.join(ROOT, "bit_weight_quantized_awq_amd", "csrc")
    exe = tmp_path / "plan_check"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}",
           os.path.join(csrc, "awq_plan.cpp"), os.path.join(ROOT, "tests", "native", "plan_check.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "plan_check ok" in res.stdout


# ------------------------------------------------- row-to-group map (g_idx)
def _dq_gidx(qw=A, qz=A, sc=A, gi=A, w=A, K=256, N=128, G=4):
    return awq.lib().awq_dequant_gidx(qw, qz, sc, gi, w, K, N, G, None)


def _gemm_gidx(x=A, qw=A, qz=A, sc=A, gi=A, bias=None, y=A, M=4, K=256, N=128, G=4):
    return awq.lib().awq_gemm_gidx(x, qw, qz, sc, gi, bias, y, M, K, N, G, None)


def _sorted(x=A, perm=A, qw=A, qz=A, sc=A, bias=None, y=A, M=4, Kin=256, rows=256, N=128,
            b=64, ws=None, wsb=0):
    return awq.lib().awq_gemm_sorted(x, perm, qw, qz, sc, bias, y, M, Kin, rows, N, b, ws, wsb,
                                     None)


@pytest.mark.parametrize("fn,kwargs,status", [
    (_dq_gidx, dict(gi=None), binding.AWQ_ERROR_INVALID_VALUE),
    (_dq_gidx, dict(G=0), binding.AWQ_ERROR_INVALID_VALUE),
    (_dq_gidx, dict(N=12), binding.AWQ_ERROR_SHAPE),
    (_dq_gidx, dict(K=65536, N=65536), binding.AWQ_ERROR_SHAPE),
    (_dq_gidx, dict(G=1 << 20, N=4096), binding.AWQ_ERROR_SHAPE),   # scales >= 2^31 elements
    (_dq_gidx, dict(gi=A + 2), binding.AWQ_ERROR_MISALIGNED),
    (_dq_gidx, dict(w=None), binding.AWQ_ERROR_INVALID_VALUE),
    (_gemm_gidx, dict(gi=None), binding.AWQ_ERROR_INVALID_VALUE),
    (_gemm_gidx, dict(G=-1), binding.AWQ_ERROR_INVALID_VALUE),
    (_gemm_gidx, dict(x=None), binding.AWQ_ERROR_INVALID_VALUE),
    (_gemm_gidx, dict(N=100), binding.AWQ_ERROR_SHAPE),
    (_gemm_gidx, dict(gi=A + 1), binding.AWQ_ERROR_MISALIGNED),
    (_gemm_gidx, dict(x=A + 1), binding.AWQ_ERROR_MISALIGNED),
    (_gemm_gidx, dict(M=0, x=None, y=None), binding.AWQ_SUCCESS),
    (_sorted, dict(perm=None), binding.AWQ_ERROR_INVALID_VALUE),
    (_sorted, dict(Kin=0), binding.AWQ_ERROR_INVALID_VALUE),
    (_sorted, dict(perm=A + 2), binding.AWQ_ERROR_MISALIGNED),
    (_sorted, dict(b=96), binding.AWQ_ERROR_SHAPE),                 # rows % block_rows
    (_sorted, dict(M=1 << 20, Kin=4096), binding.AWQ_ERROR_SHAPE),  # M * K_in >= 2^31
    (_sorted, dict(), binding.AWQ_ERROR_WORKSPACE),                 # the reordered x needs room
    (_sorted, dict(M=0, x=None, y=None), binding.AWQ_SUCCESS),
])
def test_gidx_validation(fn, kwargs, status):
    assert fn(**kwargs) == status


def test_sorted_workspace_rules():
    """The reordered x (M x rows float16) sits after the awq_gemm workspace
    of the sorted problem and never inside the fixed zero-filled region
    (4 MiB of accumulators); the call checks size and 256-byte alignment
    first."""
    fixed = 4 * 65536 * 16
    for M, rows, N, b in [(1, 8192, 7168, 128), (16, 8192, 7168, 128), (2048, 4096, 12288, 128),
                          (4, 256, 128, 64), (3, 7968, 64, 32)]:
        need = awq.sorted_workspace_size(M, rows, N, b)
        base = max(awq.gemm_workspace_size(M, rows, N, b), fixed)
        xoff = -(-base // 256) * 256
        assert need == xoff + -(-(M * rows * 2) // 256) * 256
    assert awq.sorted_workspace_size(0, 256, 128, 64) == 0
    assert awq.sorted_workspace_size(4, 256, 128, 96) == 0
    need = awq.sorted_workspace_size(4, 256, 128, 64)
    assert _sorted(ws=A, wsb=need - 1) == binding.AWQ_ERROR_WORKSPACE
    assert _sorted(ws=A + 16, wsb=need) == binding.AWQ_ERROR_MISALIGNED


def _layout_reference(g_idx, G):
    """The sorted layout restated independently: stable sort by group, then
    either whole groups (all of one power-of-two size >= 32) or 32-row
    blocks padded with -1, with one null block more when their count is
    odd."""
    import numpy as np
    g_idx = [int(v) for v in g_idx]
    K = len(g_idx)
    by_group = {}
    for k, v in enumerate(g_idx):
        by_group.setdefault(v, []).append(k)
    sizes = [len(by_group.get(v, [])) for v in range(G)]
    per = K // G if K % G == 0 else 0
    if per >= 32 and per & (per - 1) == 0 and all(c == per for c in sizes):
        perm = [k for v in range(G) for k in by_group[v]]
        return np.array(perm), np.arange(G), per
    perm, blocks = [], []
    for v in sorted(by_group):
        rows = by_group[v]
        nb = -(-len(rows) // 32)
        perm += rows + [-1] * (32 * nb - len(rows))
        blocks += [v] * nb
    if len(blocks) % 2:        # an even block count: rows a multiple of 64
        perm += [-1] * 32
        blocks += [blocks[-1]]
    return np.array(perm), np.array(blocks), 32


def test_gidx_layout_matches_reference():
    """awq_gidx_layout (host) is index work: bit-exact against the
    restatement above for uneven, empty and one-row groups, activation-order
    maps (whole groups) and activation-order maps whose group size is not a
    power of two >= 32 (blocked).  Its row order within a group is the
    oracle's stable sort."""
    import awq_inputs
    import numpy as np
    import oracle
    cases = [(awq_inputs.random_g_idx(K, G, seed), G) for K, G, seed in
             [(1, 1, 0), (7, 3, 1), (200, 7, 2), (4096, 50, 3), (300, 400, 4)]]
    cases += [(awq_inputs.act_order_g_idx(K, g, seed=K), K // g) for K, g in
              [(256, 32), (8192, 128), (14336, 128), (96, 1), (1000, 8), (4800, 96)]]
    for gi, G in cases:
        perm, blocks, b = awq.gidx_layout(gi, G)
        want_perm, want_blocks, want_b = _layout_reference(gi, G)
        np.testing.assert_array_equal(perm, want_perm)
        np.testing.assert_array_equal(blocks, want_blocks)
        assert b == want_b and len(perm) == b * len(blocks)
        order, _ = oracle.gidx_order(gi, G)
        np.testing.assert_array_equal(perm[perm >= 0], order)


def test_gidx_layout_memory_does_not_depend_on_group_count():
    """A map over a huge group range (most groups empty) sorts in O(K)
    memory and comes out blocked (three blocks and a null one, so that the
    row count is a multiple of 64)."""
    perm, blocks, b = awq.gidx_layout([3, 0, (1 << 30) - 1, 0], 1 << 30)
    assert b == 32 and blocks.tolist() == [0, 3, (1 << 30) - 1, (1 << 30) - 1]
    assert perm[:3].tolist() == [1, 3, -1] and perm[32] == 0 and perm[64] == 2
    assert len(perm) == 128 and (perm[96:] == -1).all()


@pytest.mark.parametrize("gi,G", [([0, 1, 3], 3), ([0, -1], 2), ([0, 0], 0)])
def test_gidx_layout_rejects_bad_maps(gi, G):
    with pytest.raises(binding.AwqError) as e:
        awq.gidx_layout(gi, G)
    assert e.value.status == binding.AWQ_ERROR_INVALID_VALUE


def test_gidx_layout_capacity_checked():
    import numpy as np
    g = np.array([0, 1, 0], dtype=np.int32)
    rows, b, nb = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    perm = np.zeros(63, dtype=np.int32)
    blocks = np.zeros(2, dtype=np.int32)
    st = awq.lib().awq_gidx_layout(g.ctypes.data, 3, 2, perm.ctypes.data, 63,
                                   blocks.ctypes.data, 2, ctypes.byref(rows), ctypes.byref(b),
                                   ctypes.byref(nb))
    assert st == binding.AWQ_ERROR_SHAPE and rows.value == 64 and nb.value == 2


def test_gather_rows_validation():
    lib = awq.lib()
    assert lib.awq_gather_rows(A, 256, None, A, 256, 64, None) == binding.AWQ_ERROR_INVALID_VALUE
    assert lib.awq_gather_rows(A, 0, A, A, 256, 64, None) == binding.AWQ_ERROR_INVALID_VALUE
    assert lib.awq_gather_rows(A, 256, A, A, 256, 6, None) == binding.AWQ_ERROR_SHAPE
    assert lib.awq_gather_rows(A, 256, A + 2, A, 256, 64, None) == binding.AWQ_ERROR_MISALIGNED
    assert lib.awq_gather_rows(A, 256, A, A, 1 << 30, 64, None) == binding.AWQ_ERROR_SHAPE


def _noalloc(x=A, qw=A, qz=A, sc=A, bias=None, y=A, M=4, K=256, N=128, g=64):
    return awq.lib().awq_gemm_noalloc(x, qw, qz, sc, bias, y, M, K, N, g, None)


def test_noalloc_host_checks():
    """awq_gemm_noalloc validates like awq_gemm and refuses, before any HIP
    call, a problem whose split-K workspace exceeds its fixed scratch."""
    assert _noalloc(M=0, x=None, y=None) == binding.AWQ_SUCCESS
    assert _noalloc(N=130) == binding.AWQ_ERROR_SHAPE
    assert _noalloc(g=0) == binding.AWQ_ERROR_INVALID_VALUE
    assert _noalloc(qw=None) == binding.AWQ_ERROR_INVALID_VALUE
    assert _noalloc(x=A + 1) == binding.AWQ_ERROR_MISALIGNED
    M, K, N, g = 256, 14336, 4096, 128
    assert awq.gemm_workspace_size(M, K, N, g) > binding.AWQ_NOALLOC_SCRATCH_BYTES
    assert _noalloc(M=M, K=K, N=N, g=g) == binding.AWQ_ERROR_SCRATCH
    assert "scratch" in awq.status_string(binding.AWQ_ERROR_SCRATCH)
    with awq.options(force_path="decode"):
        assert _noalloc(M=64, K=4096, N=4096, g=128) == binding.AWQ_ERROR_INVALID_VALUE


def test_workspace_need_follows_overrides():
    """An override that changes the split count changes the workspace the
    binding sizes for a shape (its per-shape memory is cleared)."""
    M, K, N, g = 1, 8192, 7168, 128
    base = binding._gemm_workspace_need(M, K, N, g)
    with awq.options(decode_steps=2):
        more = binding._gemm_workspace_need(M, K, N, g)
        assert more == awq.gemm_workspace_size(M, K, N, g) > base
    assert binding._gemm_workspace_need(M, K, N, g) == base


def test_eight_wave_decode_plan():
    """decode_waves=8 halves the split count where it applies (the LDS
    variant) and never pairs with eight steps per wave."""
    K, N, g = 8192, 7168, 128
    with awq.options(decode_waves=8, decode_steps=2):
        _, ws8 = awq.gemm_plan(1, K, N, g)
    with awq.options(decode_steps=2):
        _, ws4 = awq.gemm_plan(1, K, N, g)
    fixed = 4 * 65536 * 16
    assert (ws4 - fixed) == 2 * (ws8 - fixed) == 32 * N * 4
    with awq.options(decode_waves=8, decode_steps=8):
        _, ws = awq.gemm_plan(1, K, N, g)
    assert ws - fixed == (K // (4 * 32 * 8)) * N * 4
    with awq.options(decode_waves=8, decode_steps=4):
        _, a = awq.gemm_plan(16, K, N, g)     # the two-launch exchange too
    assert a - fixed == (K // (8 * 32 * 4)) * 16 * N * 4


def test_two_launch_exchange_takes_eight_waves_filling_one_round():
    """Batches on the two-launch exchange (above four rows, or when the atomic
    exchange would issue 380K or more atomics) run eight waves of four steps
    per work-group (half the splits) when that gives 160-256 work-groups with
    one group per wave; otherwise, and for the atomic exchange's batches, the
    four-wave plan."""
    fixed = 4 * 65536 * 16
    for M, K, N, splits in [
            (16, 14336, 4096, 14),   # 16 tiles x 14 = 224 work-groups
            (5, 14336, 4096, 14),
            (16, 8192, 7168, 8),     # 28 x 8 = 224
            (32, 8192, 7168, 8),     # two row blocks
            (16, 4096, 11008, 4),    # 43 x 4 = 172 (four waves would take 2 steps, 16 splits)
            (12, 8192, 14336, 16),   # eight waves: 448 work-groups, two rounds: four waves
            (8, 4096, 4096, 32),     # eight waves: 64 work-groups: four waves of 1 step
            (16, 4096, 7168, 16),    # g = 64 below: 4 steps would span groups
            (1, 14336, 4096, 28),    # atomic exchange, one row: eight waves of two steps, same splits
            (3, 8192, 7168, 16),     # atomic: 16 x 3 x 7168 = 344K atomics
            (4, 8192, 7168, 8),      # 16 x 4 x 7168 = 459K atomics: two launches, eight waves
            (4, 4096, 4096, 32)]:    # 524K atomics: two launches (eight waves: 64 work-groups)
        g = 64 if (M, K, N) == (16, 4096, 7168) else 128
        path, ws = awq.gemm_plan(M, K, N, g)
        assert path == binding.AWQ_PATH_DECODE
        assert ws - fixed == splits * M * N * 4, (M, K, N)


@pytest.mark.parametrize("M,K,N,g,path", [
    (17, 8192, 7168, 128, binding.AWQ_PATH_DECODE),
    (32, 8192, 7168, 128, binding.AWQ_PATH_DECODE),
    (32, 14336, 4096, -1, binding.AWQ_PATH_DECODE),
    (33, 8192, 7168, 128, binding.AWQ_PATH_PREFILL),    # above two row blocks
    (20, 4096, 4096, 64, binding.AWQ_PATH_PREFILL),     # weight below 2^25 elements
    (32, 4096, 12288, 32, binding.AWQ_PATH_PREFILL),    # one group per wave: 32 splits, partials
                                                        # above half the packed weight
    (32, 8192, 7176, 128, binding.AWQ_PATH_PREFILL),    # N % 32 != 0: no streaming variant
])
def test_plan_two_block_decode(M, K, N, g, path):
    """17-32 rows run the decode kernel's two-block form where the weight has
    at least 2^25 elements and the split partials are at most half the
    packed weight's bytes (16 * splits * M <= K); otherwise the prefill
    kernel."""
    got, ws = awq.gemm_plan(M, K, N, g)
    assert got == path
    if path == binding.AWQ_PATH_DECODE:
        splits = (ws - 4 * 65536 * 16) // (M * N * 4)
        assert ws == 4 * 65536 * 16 + splits * M * N * 4
        assert 16 * splits * M <= K


def test_plan_two_block_decode_limits():
    """Forcing the decode kernel: 33 rows cannot run it; 17-32 rows take a
    step count whose rows stay in one group (an override that would span
    groups is ignored); the fused x gather stays within one row block."""
    with awq.options(force_path="decode"):
        with pytest.raises(awq.AwqError):
            awq.gemm_plan(33, 8192, 7168, 128)
        with pytest.raises(awq.AwqError):
            awq.gemm_plan(20, 8192, 7176, 128)     # register variant: 16 rows at most
        _, ws = awq.gemm_plan(20, 4096, 7168, 64)
        assert ws == 4 * 65536 * 16 + (4096 // (4 * 32 * 2)) * 20 * 7168 * 4   # 2 steps
        with awq.options(decode_steps=4):
            _, ws4 = awq.gemm_plan(20, 4096, 7168, 64)
            assert ws4 == ws
            _, ws16 = awq.gemm_plan(16, 4096, 7168, 64)                     # one block: taken
            assert ws16 == 4 * 65536 * 16 + (4096 // (4 * 32 * 4)) * 16 * 7168 * 4
    with pytest.raises(awq.AwqError):
        awq.set_option("decode_gather_max_m", 17)
    awq.set_option("decode_gather_max_m", 16)
    awq.set_option("decode_gather_max_m", None)


@pytest.mark.parametrize("M,K,N,splits", [
    (1024, 1792, 4096, 1),    # 128-row tiles fill the CUs: no split (256 rows would split 2 ways)
    (256, 1792, 4096, 2),     # 64-row tiles, 128 of them: two splits (256 rows: three)
    (512, 4096, 4096, 2),     # 64-row tiles not taken above 256 rows: 128-row tiles, two splits
    (2048, 4096, 1536, 1),    # 128-row tiles, 192 of them: no split
    (1024, 14336, 4096, 2),   # long K keeps the split 256-row tile
    (256, 14336, 4096, 8),
])
def test_prefill_short_k_prefers_lower_tiles(M, K, N, splits):
    """With at most 64 K steps the planner trades the split 256-row tile for
    a lower one that needs fewer (or no) splits; longer K keeps the split
    tall tile.  Seen through the workspace need: the fixed exchange region
    plus one float partial plane per split, or nothing without a split."""
    path, ws = awq.gemm_plan(M, K, N, 128)
    assert path == binding.AWQ_PATH_PREFILL
    fixed = 4 * 65536 * 16
    assert ws == (fixed + splits * M * N * 4 if splits > 1 else 0), (M, K, N, ws)
