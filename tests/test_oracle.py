"""Pins of the CPU oracle against facts fixed by the page "Predibase Lorax AWQ
WQLinear" and by mathematics, independent of the oracle's own code paths.

Each pin is chosen so that a plausible slip in the oracle (nibble order,
dropped zero point, wrong group index, missing float16 rounding, transposed
operand, lost bias) fails at least one of them; test_planted_mistakes_are_caught
checks that claim by planting those slips in copies of the oracle.
"""
import json
import math
import os

import numpy as np
import pytest

import awq_inputs
import oracle
from oracle import awq_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _hex_words(rows):
    return np.array([[int(v, 16) for v in r] for r in rows], dtype=np.uint32).view(np.int32)


def _hex_f16(rows):
    return np.array([[int(v, 16) for v in r] for r in rows], dtype=np.uint16).view(np.float16)


def load_golden():
    with open(GOLDEN) as f:
        doc = json.load(f)
    out = []
    for ex in doc["examples"]:
        bias = None
        if ex["bias_f16_hex"] is not None:
            bias = _hex_f16([ex["bias_f16_hex"]])[0]
        out.append(dict(
            name=ex["name"], K=ex["K"], N=ex["N"], g=ex["group_size"],
            qweight=_hex_words(ex["qweight_hex"]),
            qzeros=_hex_words(ex["qzeros_hex"]),
            scales=_hex_f16(ex["scales_f16_hex"]),
            bias=bias,
            x=np.array(ex["x"], dtype=np.float16),
            w_bits=np.array([[int(v, 16) for v in r] for r in ex["expected_w_f16_hex"]],
                            dtype=np.uint16),
            y=np.array([[float(v) for v in r] for r in ex["expected_y"]], dtype=np.float64),
        ))
    return out


GOLDEN_CASES = load_golden()


# ----------------------------------------------------------------- golden
@pytest.mark.parametrize("ex", GOLDEN_CASES, ids=[e["name"] for e in GOLDEN_CASES])
def test_golden_dequant_bits(ex):
    w = oracle.dequant(ex["qweight"], ex["qzeros"], ex["scales"], ex["g"])
    assert w.shape == (ex["K"], ex["N"])
    np.testing.assert_array_equal(w.view(np.uint16), ex["w_bits"])


@pytest.mark.parametrize("ex", GOLDEN_CASES, ids=[e["name"] for e in GOLDEN_CASES])
def test_golden_forward_exact(ex):
    y = oracle.awq_linear_ref(ex["x"], ex["qweight"], ex["qzeros"], ex["scales"],
                              ex["bias"], ex["g"])
    np.testing.assert_array_equal(y, ex["y"])
    y2 = oracle.awq_linear_loops(ex["x"], ex["qweight"], ex["qzeros"], ex["scales"],
                                 ex["bias"], ex["g"])
    np.testing.assert_array_equal(y2, ex["y"])


# ------------------------------------------------------- pack / unpack
def test_pack_single_nibble_positions():
    """Every value at every position lands in bits 4j..4j+3 (closed form)."""
    for j in range(8):
        for v in range(16):
            q = np.zeros((1, 8), dtype=np.int64)
            q[0, j] = v
            word = oracle.pack_int4(q).view(np.uint32)[0, 0]
            assert int(word) == (v << (4 * j))
            back = oracle.unpack_int4(oracle.pack_int4(q))
            np.testing.assert_array_equal(back, q)


def test_pack_unpack_roundtrip_random():
    rng = np.random.default_rng(123)
    q = rng.integers(0, 16, size=(37, 64))
    p = oracle.pack_int4(q)
    assert p.dtype == np.int32 and p.shape == (37, 8)
    np.testing.assert_array_equal(oracle.unpack_int4(p), q)
    words = rng.integers(0, 2 ** 32, size=(19, 5), dtype=np.uint32).view(np.int32)
    words[0, 0] = np.uint32(0xFFFFFFFF).view(np.int32)   # all bits set
    words[0, 1] = np.uint32(0x80000000).view(np.int32)   # only bit 31
    np.testing.assert_array_equal(oracle.pack_int4(oracle.unpack_int4(words)), words)
    assert oracle.unpack_int4(words[:1, :2]).tolist() == [[15] * 8 + [0] * 7 + [8]]


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.pack_int4(np.full((1, 8), 16))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.zeros((1, 7), dtype=np.int64))


# ------------------------------------------------------------- dequant
def test_dequant_every_pair_every_float16_scale():
    """All (q, z) in 0..15 x 0..15 against every finite float16 scale of
    either sign, compared bit for bit with numpy's float16 multiply (an
    independent library routine: it rounds the exact product once)."""
    pos = np.arange(0x0000, 0x7C00, dtype=np.uint16)
    finite = np.concatenate([pos, pos | np.uint16(0x8000)])       # 63488 values
    N = finite.size
    assert N % 8 == 0
    qs, zs = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    qs, zs = qs.ravel(), zs.ravel()                                 # 256 pairs
    K = qs.size
    qweight = np.repeat((qs.astype(np.uint32) * np.uint32(0x11111111))[:, None],
                        N // 8, axis=1).view(np.int32)
    qzeros = np.repeat((zs.astype(np.uint32) * np.uint32(0x11111111))[:, None],
                       N // 8, axis=1).view(np.int32)
    scales = np.repeat(finite.view(np.float16)[None, :], K, axis=0)
    w = oracle.dequant(qweight, qzeros, scales, 1)                 # one group per row
    with np.errstate(over="ignore"):
        expect = (qs - zs).astype(np.float16)[:, None] * scales     # float16 arithmetic
    np.testing.assert_array_equal(w.view(np.uint16), expect.view(np.uint16))


def test_dequant_float32_route_agrees():
    """(q - z) * s in float32 then one cast also matches: the product of a
    4-bit integer and a float16 is exact in float32."""
    p = awq_inputs.make_inputs(1, 64, 256, 16, seed=7, scale_lo=-3.0, scale_hi=3.0)
    w = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], 16)
    q = np.stack([(p["qweight"].view(np.uint32) >> (4 * j)) & 0xF for j in range(8)], -1)
    z = np.stack([(p["qzeros"].view(np.uint32) >> (4 * j)) & 0xF for j in range(8)], -1)
    q = q.reshape(64, 256).astype(np.float32)
    z = np.repeat(z.reshape(4, 256), 16, axis=0).astype(np.float32)
    s = np.repeat(p["scales"].astype(np.float32), 16, axis=0)
    np.testing.assert_array_equal(w.view(np.uint16), ((q - z) * s).astype(np.float16).view(np.uint16))


# ----------------------------------------------------------------- GEMM
@pytest.mark.parametrize("M,K,N,g,bias", [
    (1, 8, 8, 1, False), (3, 16, 16, 4, True), (2, 24, 8, 8, True),
    (2, 16, 24, -1, False), (1, 32, 16, 16, True), (3, 12, 8, 3, False)])
def test_tiny_bruteforce_loops(M, K, N, g, bias):
    p = awq_inputs.make_inputs(M, K, N, g, seed=M * 100 + K + N, scale_lo=-0.5,
                               scale_hi=0.5, bias=bias)
    ref = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    loops = oracle.awq_linear_loops(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    np.testing.assert_allclose(ref, loops, rtol=1e-12, atol=1e-12)


def _equal_q_z(K, N, g, seed):
    rng = np.random.default_rng(seed)
    G = K // (K if g == -1 else g)
    qzeros = rng.integers(0, 2 ** 32, size=(G, N // 8), dtype=np.uint32).view(np.int32)
    gg = K if g == -1 else g
    qweight = np.repeat(qzeros, gg, axis=0)        # q == z everywhere
    return qweight, qzeros


@pytest.mark.parametrize("g", [1, 4, 32, -1])
def test_q_equal_z_gives_bias_exactly(g):
    K, N, M = 32, 40, 3
    qweight, qzeros = _equal_q_z(K, N, g, 5)
    p = awq_inputs.make_inputs(M, K, N, g, seed=6, scale_lo=-2, scale_hi=2, bias=True)
    y0 = oracle.awq_linear_ref(p["x"], qweight, qzeros, p["scales"], None, g)
    assert np.all(y0 == 0.0)
    y1 = oracle.awq_linear_ref(p["x"], qweight, qzeros, p["scales"], p["bias"], g)
    np.testing.assert_array_equal(y1, np.broadcast_to(p["bias"].astype(np.float64), (M, N)))


def test_group_minus_one_equals_single_group():
    p = awq_inputs.make_inputs(5, 96, 48, -1, seed=11, bias=True)
    a = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], -1)
    b = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], 96)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(
        oracle.dequant(p["qweight"], p["qzeros"], p["scales"], -1).view(np.uint16),
        oracle.dequant(p["qweight"], p["qzeros"], p["scales"], 96).view(np.uint16))


def test_one_hot_rows_select_dequant_rows():
    K, N, g = 64, 32, 16
    p = awq_inputs.make_inputs(1, K, N, g, seed=12)
    ks = [0, 5, 15, 16, 63]
    x = np.zeros((len(ks), K), dtype=np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = oracle.awq_linear_ref(x, p["qweight"], p["qzeros"], p["scales"], None, g)
    w = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    np.testing.assert_array_equal(y, w[ks].astype(np.float64))


def test_closed_form_constant_difference_power_of_two_scale():
    """q - z == c everywhere and s == 2^e: y[m, n] = c * 2^e * sum_k x[m, k]."""
    K, N, M, g = 48, 16, 4, 8
    c, e = -5, -3
    zn, qn = 9, 9 + c
    qweight = np.full((K, N // 8), np.uint32(qn * 0x11111111), dtype=np.uint32).view(np.int32)
    qzeros = np.full((K // g, N // 8), np.uint32(zn * 0x11111111), dtype=np.uint32).view(np.int32)
    scales = np.full((K // g, N), 2.0 ** e, dtype=np.float16)
    x = np.random.default_rng(3).standard_normal((M, K)).astype(np.float16)
    y = oracle.awq_linear_ref(x, qweight, qzeros, scales, None, g)
    for m in range(M):
        expect = c * 2.0 ** e * math.fsum(float(v) for v in x[m])
        assert np.all(y[m] == expect)


def test_linearity_and_leading_dims():
    p = awq_inputs.make_inputs(6, 32, 16, 8, seed=21, bias=True)
    x = p["x"].astype(np.float64)
    f = lambda v, b: oracle.awq_linear_ref(v, p["qweight"], p["qzeros"], p["scales"], b, 8)
    np.testing.assert_allclose(f(x[:3] + 2 * x[3:], None), f(x[:3], None) + 2 * f(x[3:], None),
                               rtol=1e-12, atol=1e-12)
    y3 = f(p["x"].reshape(2, 3, 32), p["bias"])
    assert y3.shape == (2, 3, 16)
    np.testing.assert_array_equal(y3.reshape(6, 16), f(p["x"], p["bias"]))


# -------------------------------------------------------------- validate
def test_validate_rules():
    assert oracle.validate(4, 128, (256, 16)) == (256, 128, 128, 2)
    assert oracle.validate(4, -1, (256, 16)) == (256, 128, 256, 1)
    with pytest.raises(ValueError):
        oracle.validate(8, 128, (256, 16))       # only 4-bit
    with pytest.raises(ValueError):
        oracle.validate(4, 100, (256, 16))       # K % g
    with pytest.raises(ValueError):
        oracle.validate(4, 0, (256, 16))
    with pytest.raises(ValueError):
        oracle.validate(4, -2, (256, 16))
    with pytest.raises(ValueError):
        oracle.validate(4, 128, (256, 16), qzeros_shape=(2, 15))
    with pytest.raises(ValueError):
        oracle.validate(4, 128, (256, 16), scales_shape=(2, 120))
    with pytest.raises(ValueError):
        oracle.validate(4, 128, (256, 16), bias_shape=(127,))


# ------------------------------------------------------ planted mistakes
def _golden_pins_pass(dequant_fn):
    """Golden dequant bits and golden forward values for a dequant variant."""
    for ex in GOLDEN_CASES:
        w = dequant_fn(ex["qweight"], ex["qzeros"], ex["scales"], ex["g"])
        if w.shape != ex["w_bits"].shape or not np.array_equal(
                np.asarray(w, dtype=np.float16).view(np.uint16), ex["w_bits"]):
            return False
        y = ex["x"].astype(np.float64) @ np.asarray(w, dtype=np.float64)
        if ex["bias"] is not None:
            y = y + ex["bias"].astype(np.float64)
        if not np.array_equal(y, ex["y"]):
            return False
    return True


def _q_equal_z_pin_passes(dequant_fn):
    qweight, qzeros = _equal_q_z(32, 16, 8, 5)
    scales = np.full((4, 16), 0.5, dtype=np.float16)
    return np.all(np.asarray(dequant_fn(qweight, qzeros, scales, 8), dtype=np.float64) == 0)


def test_planted_mistakes_are_caught():
    """Copies of the oracle's dequant with one plausible slip each must fail
    the golden pins (and the unmodified one must pass them)."""
    assert _golden_pins_pass(oracle.dequant)
    assert _q_equal_z_pin_passes(oracle.dequant)

    def unpack_msb_first(p):
        u = p.view(np.uint32).astype(np.int64)
        out = np.empty((u.shape[0], u.shape[1] * 8), dtype=np.int64)
        for j in range(8):
            out[:, j::8] = (u >> (4 * (7 - j))) & 0xF
        return out

    def make(unpack=awq_oracle.unpack_int4, grp=lambda K, g, G: np.arange(K) // g,
             zero=True, round16=True, sign=1):
        def dq(qweight, qzeros, scales, group_size):
            K = qweight.shape[0]
            g = K if group_size == -1 else group_size
            G = K // g
            gi = grp(K, g, G)
            q = unpack(qweight)
            z = unpack(qzeros)[gi] if zero else 0
            d = sign * (q - z).astype(np.float64) * scales.astype(np.float64)[gi]
            return d.astype(np.float16) if round16 else d
        return dq

    assert _golden_pins_pass(make())                                   # control
    assert not _golden_pins_pass(make(unpack=unpack_msb_first))       # nibble order
    assert not _golden_pins_pass(make(grp=lambda K, g, G: np.arange(K) % G))  # group index
    assert not _golden_pins_pass(make(round16=False))                  # no float16 rounding
    assert not _golden_pins_pass(make(sign=-1))                        # z - q
    assert not _golden_pins_pass(make(zero=False))                     # zero point dropped
    assert not _q_equal_z_pin_passes(make(zero=False))


def test_planted_forward_mistakes_are_caught():
    ex = GOLDEN_CASES[0]
    w = oracle.dequant(ex["qweight"], ex["qzeros"], ex["scales"], ex["g"]).astype(np.float64)
    x = ex["x"].astype(np.float64)
    good = x @ w + ex["bias"].astype(np.float64)
    np.testing.assert_array_equal(good, ex["y"])
    assert not np.array_equal(x @ w, ex["y"])                          # bias lost
    assert not np.array_equal(x[::-1] @ w + ex["bias"].astype(np.float64), ex["y"])  # rows swapped


# --------------------------------------------------------------- inputs
def test_input_generator_shapes_and_prefix():
    a = awq_inputs.workload_inputs("decode_sweep_k8192_n7168", 4)
    b = awq_inputs.workload_inputs("decode_sweep_k8192_n7168", 16)
    assert a["qweight"].shape == (8192, 896) and a["qweight"].dtype == np.int32
    assert a["qzeros"].shape == (64, 896) and a["scales"].shape == (64, 7168)
    assert a["scales"].dtype == np.float16 and a["x"].dtype == np.float16
    np.testing.assert_array_equal(a["qweight"], b["qweight"])
    np.testing.assert_array_equal(a["x"], b["x"][:4])
    t = awq_inputs.workload_inputs("tiny_m4_k256_n128", 4)
    assert t["qweight"].shape == (256, 16) and t["qzeros"].shape == (4, 16)
    assert t["scales"].shape == (4, 128) and t["bias"].shape == (128,)
    assert 0.002 <= float(t["scales"].min()) and float(t["scales"].max()) <= 0.02
    d = awq_inputs.workload_inputs("mlp_down_k14336_n4096", 1, group_size=-1)
    assert d["qzeros"].shape == (1, 512) and d["scales"].shape == (1, 4096)
    # uniform nibbles: every value 0..15 appears with frequency ~1/16
    nib = oracle.unpack_int4(t["qweight"])
    counts = np.bincount(nib.ravel(), minlength=16) / nib.size
    assert np.all(np.abs(counts - 1 / 16) < 0.01)


# ----------------------------------------------- the unquantised baseline
def test_dense_linear_pins():
    """F.linear(x, w, b) = x . w^T + b (page "Predibase Lorax Linear Layer
    Factory", Description: FastLinear).  Pinned by: the pure-Python loop on a
    tiny case; an identity weight returning x exactly; one-hot rows selecting
    the columns of w^T bit for bit; and the identity F.linear(x, W^T) = x . W
    against the independently pinned quantised forward, whose dequantised
    weight is (K, N) where F.linear's is (N, K) -- a transposed operand fails
    here."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 5)).astype(np.float16)
    w = rng.standard_normal((4, 5)).astype(np.float16)
    b = rng.standard_normal(4).astype(np.float16)
    np.testing.assert_allclose(oracle.dense_linear_ref(x, w, b),
                               oracle.dense_linear_loops(x, w, b), rtol=1e-12, atol=1e-12)
    eye = np.eye(6, dtype=np.float16)
    xs = rng.standard_normal((2, 6)).astype(np.float16)
    np.testing.assert_array_equal(oracle.dense_linear_ref(xs, eye, None), xs.astype(np.float64))
    w2 = rng.standard_normal((7, 9)).astype(np.float16)
    onehot = np.zeros((3, 9), dtype=np.float16)
    ks = [0, 4, 8]
    onehot[np.arange(3), ks] = 1.0
    np.testing.assert_array_equal(oracle.dense_linear_ref(onehot, w2, None),
                                  w2.T[ks].astype(np.float64))
    p = awq_inputs.make_inputs(2, 64, 24, 32, seed=9, bias=True)
    wq = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], 32)      # (K, N)
    np.testing.assert_allclose(oracle.dense_linear_ref(p["x"], wq.T, p["bias"]),
                               oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"],
                                                     p["scales"], p["bias"], 32),
                               rtol=1e-12, atol=1e-12)
    with pytest.raises(AssertionError):
        # a transposed weight (read as (K, N)) must not pass the same check
        np.testing.assert_allclose(oracle.dense_linear_loops(p["x"][:, :24], wq[:24, :24], None),
                                   oracle.dense_linear_ref(p["x"][:, :24], wq[:24, :24].T, None),
                                   rtol=1e-6, atol=1e-6)


# ------------------------------------------------ row-to-group map (g_idx)
def test_gidx_contiguous_map_is_the_grouped_dequant():
    """g_idx[k] = k // g is the contiguous grouping: bit-identical to the
    independently pinned grouped dequantisation, and the worked examples'
    weights come out bit for bit through the map."""
    for g in (1, 4, 32, 64):
        p = awq_inputs.make_inputs(1, 64, 24, g, seed=20 + g)
        gi = np.arange(64) // g
        np.testing.assert_array_equal(
            oracle.dequant_gidx(p["qweight"], p["qzeros"], p["scales"], gi).view(np.uint16),
            oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g).view(np.uint16))
    for ex in GOLDEN_CASES:
        K = ex["K"]
        g = K if ex["g"] == -1 else ex["g"]
        w = oracle.dequant_gidx(ex["qweight"], ex["qzeros"], ex["scales"], np.arange(K) // g)
        np.testing.assert_array_equal(w.view(np.uint16), ex["w_bits"])


def test_gidx_constant_map_is_one_group():
    p = awq_inputs.make_inputs(2, 48, 16, -1, seed=31)
    np.testing.assert_array_equal(
        oracle.dequant_gidx(p["qweight"], p["qzeros"], p["scales"], np.zeros(48, np.int32)),
        oracle.dequant(p["qweight"], p["qzeros"], p["scales"], -1))


def test_gidx_act_order_is_a_row_permutation_of_grouped():
    """An activation-ordered weight is a grouped weight whose input rows were
    shuffled: with perm a permutation of the rows, qweight_p = qweight[perm]
    and g_idx = perm // g, every dequantised row k equals the grouped row
    perm[k] bit for bit, and x[:, perm] through the map gives the grouped
    forward of x (the same terms summed in another order)."""
    K, N, g = 96, 32, 16
    p = awq_inputs.make_inputs(3, K, N, g, seed=41, bias=True)
    perm = np.random.default_rng(42).permutation(K)
    qw_p = p["qweight"][perm]
    gi = perm // g
    w_grouped = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)
    w_map = oracle.dequant_gidx(qw_p, p["qzeros"], p["scales"], gi)
    np.testing.assert_array_equal(w_map.view(np.uint16), w_grouped[perm].view(np.uint16))
    y_map = oracle.awq_linear_gidx_ref(p["x"][:, perm], qw_p, p["qzeros"], p["scales"], gi,
                                       p["bias"])
    y_grp = oracle.awq_linear_ref(p["x"], p["qweight"], p["qzeros"], p["scales"], p["bias"], g)
    np.testing.assert_allclose(y_map, y_grp, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("M,K,N,G,bias", [(2, 16, 8, 3, True), (1, 24, 16, 5, False)])
def test_gidx_tiny_bruteforce_loops(M, K, N, G, bias):
    """Arbitrary maps (unequal, possibly empty groups) against the
    pure-Python loop."""
    p = awq_inputs.make_inputs(M, K, N, -1, seed=K + G, bias=bias)
    rng = np.random.default_rng(K * G)
    qz = rng.integers(0, 2 ** 32, size=(G, N // 8), dtype=np.uint32).view(np.int32)
    sc = rng.uniform(0.001, 0.01, size=(G, N)).astype(np.float16)
    gi = awq_inputs.random_g_idx(K, G, seed=G)
    ref = oracle.awq_linear_gidx_ref(p["x"], p["qweight"], qz, sc, gi, p["bias"])
    loops = oracle.awq_linear_gidx_loops(p["x"].tolist(), p["qweight"].tolist(), qz.tolist(),
                                         sc.tolist(), gi.tolist(),
                                         None if p["bias"] is None else p["bias"].tolist())
    np.testing.assert_allclose(ref, loops, rtol=1e-12, atol=1e-12)


def test_gidx_validation():
    with pytest.raises(ValueError):
        oracle.validate_gidx(np.array([0, 1, 3]), 3, 3)        # entry >= G
    with pytest.raises(ValueError):
        oracle.validate_gidx(np.array([0, -1, 1]), 3, 3)       # negative entry
    with pytest.raises(ValueError):
        oracle.validate_gidx(np.array([0, 1]), 3, 3)           # wrong length
    with pytest.raises(ValueError):
        oracle.validate_gidx(np.array([0.0, 1.0, 2.0]), 3, 3)  # not integers
    p = awq_inputs.make_inputs(1, 16, 8, 4, seed=1)
    with pytest.raises(ValueError):                            # scales rows != zero rows
        oracle.dequant_gidx(p["qweight"], p["qzeros"], p["scales"][:3], np.zeros(16, np.int32))


def test_gidx_order_is_a_stable_sort_by_group():
    """gidx_order: a permutation of the rows under which the map is
    non-decreasing, rows of one group kept in input order, and group sizes
    that count the rows; on an activation-ordered map every group holds g
    rows, so the sorted map is exactly j // g."""
    gi = awq_inputs.random_g_idx(200, 7, seed=3)
    perm, counts = oracle.gidx_order(gi, 7)
    assert sorted(perm.tolist()) == list(range(200))
    s = gi[perm]
    assert np.all(np.diff(s) >= 0)
    for grp in range(7):
        rows = perm[s == grp]
        assert np.all(np.diff(rows) > 0)
        assert counts[grp] == np.count_nonzero(gi == grp)
    ao = awq_inputs.act_order_g_idx(256, 32, seed=5)
    perm, counts = oracle.gidx_order(ao, 8)
    np.testing.assert_array_equal(ao[perm], np.arange(256) // 32)
    assert np.all(counts == 32)


def test_gidx_planted_mistakes_are_caught():
    """Copies of dequant_gidx with one slip each fail the permutation pin:
    ignoring the map (contiguous groups), indexing the packed weight rows
    through the map, or taking the zero row from the map but the scale row
    from k // g."""
    K, N, g = 64, 16, 16
    p = awq_inputs.make_inputs(1, K, N, g, seed=7)
    perm = np.random.default_rng(8).permutation(K)
    qw_p, gi = p["qweight"][perm], perm // g
    want = oracle.dequant(p["qweight"], p["qzeros"], p["scales"], g)[perm].view(np.uint16)

    def make(slip):
        def dq(qweight, qzeros, scales, g_idx):
            q = oracle.unpack_int4(qweight)
            z = oracle.unpack_int4(qzeros)
            kk = np.arange(qweight.shape[0])
            zr, sr = g_idx, g_idx
            if slip == "ignore":
                zr = sr = kk // g
            elif slip == "scale_contiguous":
                sr = kk // g
            elif slip == "weight_rows":
                q = q[g_idx]
            d = (q - z[zr]).astype(np.float64) * scales.astype(np.float64)[sr]
            return d.astype(np.float16)
        return dq

    assert np.array_equal(make(None)(qw_p, p["qzeros"], p["scales"], gi).view(np.uint16), want)
    for slip in ("ignore", "scale_contiguous", "weight_rows"):
        got = make(slip)(qw_p, p["qzeros"], p["scales"], gi).view(np.uint16)
        assert not np.array_equal(got, want), slip
