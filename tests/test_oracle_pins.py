"""Pins of the CPU oracle against closed forms, invariants, library routines and
brute force: nothing here compares the oracle with itself.

The pages ("Doubling LLM token rates in ComfyUI", section "Optimizing the
Linear Kernel") print no worked numeric example, so every expected value below
follows from the stated definitions: W4A8/W6A8 codes with per-group scales,
per-token int8 activation quantisation, exact integer dot products, rescale to
bf16.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth
from tests.codes import (bf16_to_f64, f64_to_bf16_bits_via_f32, pack, pack_w4, pack_w6,
                         random_codes)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- number formats

def test_f16_decode_matches_numpy_for_every_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(p)) for p in pats[::7]])
    r = ref[::7]
    fin = np.isfinite(r)
    assert np.array_equal(got[fin], r[fin])
    assert np.array_equal(np.isnan(got), np.isnan(r))


def test_bf16_rounding_fixed_cases():
    # 1 + 2^-8 is the midpoint of 1.0 (0x3F80) and 1 + 2^-7 (0x3F81): ties go to even.
    assert oracle.f64_to_bf16(1 + 2 ** -8) == 0x3F80
    # 1 + 3*2^-8 is the midpoint of 0x3F81 and 0x3F82: even is 0x3F82.
    assert oracle.f64_to_bf16(1 + 3 * 2 ** -8) == 0x3F82
    # Just above a midpoint rounds up; via fp32 it would first collapse onto the midpoint.
    assert oracle.f64_to_bf16(1 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert oracle.f64_to_bf16(-2.0) == 0xC000
    assert oracle.f64_to_bf16(0.0) == 0x0000
    assert oracle.f64_to_bf16(3.5e38) == 0x7F80          # beyond the largest finite bf16
    assert oracle.f64_to_bf16(-3.5e38) == 0xFF80


def test_bf16_rounding_matches_fp32_bit_rounding():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 6, 4000)).astype(np.float32)
    ref = f64_to_bf16_bits_via_f32(v.astype(np.float64))
    got = np.array([oracle.f64_to_bf16(float(x)) for x in v], np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- weight codes

def test_w4_fixed_example():
    # Byte 0x8F: low nibble 0xF is -1 (even k), high nibble 0x8 is -8 (odd k).
    w = oracle.decode(4, np.array([[0x8F]], np.uint8), 2)
    assert w.tolist() == [[-1, -8]]


def test_w6_fixed_example():
    # (-1, 0, -32, 31) -> 24-bit word 0x3F | 0<<6 | 0x20<<12 | 0x1F<<18 = 0x7E003F -> bytes 3F 00 7E.
    b = pack_w6(np.array([[-1, 0, -32, 31]]))
    assert b.tolist() == [[0x3F, 0x00, 0x7E]]
    assert oracle.decode(6, b, 4).tolist() == [[-1, 0, -32, 31]]


def test_every_w4_byte():
    b = np.arange(256, dtype=np.uint8).reshape(256, 1)
    w = oracle.decode(4, b, 2)
    lo = np.arange(256) & 0xF
    hi = np.arange(256) >> 4
    assert np.array_equal(w[:, 0], np.where(lo >= 8, lo - 16, lo))
    assert np.array_equal(w[:, 1], np.where(hi >= 8, hi - 16, hi))


@pytest.mark.parametrize("bits", [4, 6])
def test_every_code_in_every_position(bits):
    lo, hi = (-8, 7) if bits == 4 else (-32, 31)
    vals = np.arange(lo, hi + 1)
    per = 2 if bits == 4 else 4
    K = per * 4
    rows = []
    for pos in range(per):
        for v in vals:
            r = np.zeros(K, np.int64)
            r[pos] = v
            r[per + (pos + 1) % per] = -1 - v if bits == 4 and -1 - v >= lo else 0
            rows.append(r)
    codes = np.array(rows)
    assert np.array_equal(oracle.decode(bits, pack(bits, codes), K), codes)


# ---------------------------------------------------------------- activation quantisation

def _bf16(vals):
    return f64_to_bf16_bits_via_f32(np.asarray(vals, np.float64))


def test_quant_round_half_even():
    # amax 127 gives s = 127/127 = 1 exactly, so q = rint(x): halves go to even.
    x = _bf16([[127.0, 2.5, -2.5, 0.5, 1.5, -0.5, 126.5, 0.0]])
    q, s = oracle.quantize_act(x)
    assert s.tolist() == [1.0]
    assert q.tolist() == [[127, 2, -2, 0, 2, 0, 126, 0]]


def test_quant_zero_row_and_single_nonzero():
    x = np.zeros((2, 128), np.uint16)
    x[1, 17] = _bf16([[-3.0]])[0, 0]
    q, s = oracle.quantize_act(x)
    assert s[0] == 0.0 and not q[0].any()
    assert s[1] == np.float32(3.0) / np.float32(127.0)
    assert q[1, 17] == -127 and np.count_nonzero(q[1]) == 1


def _check_quant_invariants(x):
    q, s = oracle.quantize_act(x)
    xf = bf16_to_f64(x)
    amax = np.abs(xf).max(axis=1)
    assert np.all(np.abs(q.astype(int)) <= 127)
    for m in range(x.shape[0]):
        if amax[m] == 0:
            assert s[m] == 0 and not q[m].any()
            continue
        assert s[m] == np.float32(np.float32(amax[m]) / np.float32(127.0))
        am = np.argmax(np.abs(xf[m]))
        assert abs(int(q[m, am])) == 127
        assert np.all((np.sign(q[m]) == np.sign(xf[m])) | (q[m] == 0))
        err = np.abs(xf[m] - q[m].astype(np.float64) * float(s[m]))
        assert np.all(err <= float(s[m]) * (0.5 + 2.0 ** -17))


def test_quant_invariants_random():
    rng = np.random.default_rng(1)
    x = synth.f32_to_bf16_bits((rng.standard_normal((4, 4096)) * [[1], [1e-3], [300], [7]]).astype(np.float32))
    _check_quant_invariants(x)


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 4), st.integers(1, 300), st.integers(0, 2 ** 31), st.floats(1e-3, 1e3))
def test_quant_invariants_property(M, K, seed, scale):
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) * scale).astype(np.float32))
    _check_quant_invariants(x)


@pytest.mark.parametrize("j", [-20, -3, 1, 9])
def test_quant_power_of_two_scaling(j):
    x = synth.activations(3, 512, seed=11)
    xs = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * np.float32(2.0 ** j))
    q0, s0 = oracle.quantize_act(x)
    q1, s1 = oracle.quantize_act(xs)
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, (s0.astype(np.float64) * 2.0 ** j).astype(np.float32))


# ---------------------------------------------------------------- integer dot products

@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 5, 256), (4, 16, 512)])
def test_group_acc_equals_int64_sums(bits, M, N, K):
    rng = np.random.default_rng(M * 100 + N + K)
    codes = random_codes(rng, bits, N, K)
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    acc = oracle.group_acc(bits, q, pack(bits, codes))
    ref = np.einsum("mgk,ngk->mng", q.astype(np.int64).reshape(M, K // 128, 128),
                    codes.astype(np.int64).reshape(N, K // 128, 128))
    assert np.array_equal(acc.astype(np.int64), ref)


@pytest.mark.parametrize("bits,c", [(4, -8), (4, 7), (6, -32), (6, 31), (6, -1)])
@pytest.mark.parametrize("d", [-127, 127, 5])
def test_group_acc_constant(bits, c, d):
    K = 384
    codes = np.full((3, K), c)
    q = np.full((2, K), d, np.int8)
    acc = oracle.group_acc(bits, q, pack(bits, codes))
    assert np.all(acc == 128 * c * d)


@pytest.mark.parametrize("bits", [4, 6])
def test_group_acc_one_hot(bits):
    rng = np.random.default_rng(3)
    K, N = 512, 7
    codes = random_codes(rng, bits, N, K)
    for k0 in (0, 1, 127, 128, 255, 383, 511):
        q = np.zeros((1, K), np.int8)
        q[0, k0] = -93
        acc = oracle.group_acc(bits, q, pack(bits, codes))
        g0 = k0 // 128
        assert np.array_equal(acc[0, :, g0], -93 * codes[:, k0])
        mask = np.ones(K // 128, bool)
        mask[g0] = False
        assert not acc[0][:, mask].any()


def test_group_acc_bounds_at_extremes():
    K = 128
    for bits, c, bound in ((4, -8, 130048), (6, -32, 520192)):
        codes = np.full((1, K), c)
        q = np.full((1, K), -127, np.int8)
        acc = oracle.group_acc(bits, q, pack(bits, codes))
        assert acc[0, 0, 0] == 127 * -c * 128 and abs(int(acc[0, 0, 0])) <= bound


# ---------------------------------------------------------------- rescale and output rounding

@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (16, 512)])
def test_linear_matches_float64_dequant_then_matmul(bits, M, N, K):
    rng = np.random.default_rng(bits * 1000 + M * 10 + N + K)
    codes = random_codes(rng, bits, N, K)
    S = rng.uniform(0.005, 0.02, size=(N, K // 128)).astype(np.float16)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    q, s = oracle.quantize_act(x)
    y, pre = oracle.linear(bits, q, s, pack(bits, codes), S, want_pre=True)
    a = q.astype(np.float64) * s.astype(np.float64)[:, None]
    w = codes.astype(np.float64) * np.repeat(S.astype(np.float64), 128, axis=1)
    ref = a @ w.T
    terms = np.abs(a) @ np.abs(w).T
    assert np.all(np.abs(pre - ref) <= 1e-12 * terms + 1e-300)
    # y is the nearest bf16 to pre: neither neighbour is strictly closer.
    yv = bf16_to_f64(y)
    up = bf16_to_f64((y.astype(np.int32) + 1).astype(np.uint16))
    dn = bf16_to_f64((y.astype(np.int32) - 1).astype(np.uint16))
    d0 = np.abs(yv - pre)
    assert np.all(d0 <= np.abs(up - pre)) and np.all(d0 <= np.abs(dn - pre))


@pytest.mark.parametrize("bits", [4, 6])
def test_linear_integer_special_case(bits):
    # S == 1 and integer-valued x with amax 127: s = 1, q = x, y = bf16(q @ w^T) exactly.
    rng = np.random.default_rng(9)
    M, N, K = 3, 24, 640
    codes = random_codes(rng, bits, N, K)
    xi = rng.integers(-127, 128, size=(M, K))
    xi[:, 5] = 127
    x = _bf16(xi.astype(np.float64))
    q, s = oracle.quantize_act(x)
    assert np.all(s == 1.0) and np.array_equal(q.astype(np.int64), xi)
    S = np.ones((N, K // 128), np.float16)
    y = oracle.linear(bits, q, s, pack(bits, codes), S)
    ref = xi.astype(np.int64) @ codes.astype(np.int64).T
    assert np.array_equal(y, f64_to_bf16_bits_via_f32(ref.astype(np.float64)))


def test_linear_zero_row_gives_zero():
    rng = np.random.default_rng(2)
    canon, S = synth.weights(4, 8, 256, seed=4)
    x = synth.activations(2, 256, seed=3)
    x[1] = 0
    q, s = oracle.quantize_act(x)
    y = oracle.linear(4, q, s, canon, S)
    assert not y[1].any() and y[0].any()


@pytest.mark.parametrize("bits", [4, 6])
def test_rows_are_independent(bits):
    canon, S = synth.weights(bits, 40, 512, seed=21)
    x = synth.activations(3, 512)
    q, s = oracle.quantize_act(x)
    y3 = oracle.linear(bits, q, s, canon, S)
    for m in range(3):
        qm, sm = oracle.quantize_act(x[m:m + 1])
        assert np.array_equal(oracle.linear(bits, qm, sm, canon, S), y3[m:m + 1])


# ---------------------------------------------------------------- weightless RMSNorm prologue

def test_rmsnorm_small_closed_forms():
    # K = 4, x = (1, -1, 3, -3): mean square 5; t = x / sqrt(5 + 1e-6).
    x = _bf16([[1.0, -1.0, 3.0, -3.0]])
    t = bf16_to_f64(oracle.rmsnorm_bf16(x))
    ref = np.array([1, -1, 3, -3]) / np.sqrt(5 + 1e-6)
    assert np.all(np.abs(t - ref) <= 2 ** -8 * np.abs(ref))
    # A divisor of K-1 instead of K would give sqrt(20/3): about 15% off, caught above.
    # Tiny x: the 1e-6 in the root matters.  x = 1e-3 (as bf16): t = x / sqrt(x^2 + 1e-6).
    xs = synth.f32_to_bf16_bits(np.full((1, 4), 1e-3, np.float32))
    xv = bf16_to_f64(xs)[0, 0]
    t = bf16_to_f64(oracle.rmsnorm_bf16(xs))
    ref = xv / np.sqrt(xv * xv + 1e-6)
    assert np.all(np.abs(t - ref) <= 2 ** -8 * ref)
    assert abs(ref - 1.0) > 0.2


def test_rmsnorm_random_rows():
    rng = np.random.default_rng(8)
    x = synth.f32_to_bf16_bits((rng.standard_normal((3, 1000)) * [[0.01], [1], [50]]).astype(np.float32))
    xf = bf16_to_f64(x)
    ref = xf / np.sqrt((xf ** 2).mean(axis=1, keepdims=True) + 1e-6)
    t = bf16_to_f64(oracle.rmsnorm_bf16(x))
    assert np.all(np.abs(t - ref) <= 2 ** -8 * np.abs(ref) + 1e-30)


# ---------------------------------------------------------------- weighted RMSNorm and SwiGLU prologues

def test_wrmsnorm_unit_weights_is_the_weightless_norm():
    rng = np.random.default_rng(21)
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, 640)).astype(np.float32))
    ones = synth.f32_to_bf16_bits(np.ones(640, np.float32))
    assert np.array_equal(oracle.wrmsnorm_bf16(x, ones), oracle.rmsnorm_bf16(x))


@pytest.mark.parametrize("j", [-3, 1, 4])
def test_wrmsnorm_power_of_two_weights_scale_exactly(j):
    # w = 2^j everywhere: every t is 2^j times the weightless one, exactly
    # (scaling by a power of two commutes with both roundings away from overflow)
    rng = np.random.default_rng(22 + j)
    x = synth.f32_to_bf16_bits(rng.standard_normal((2, 256)).astype(np.float32))
    w = synth.f32_to_bf16_bits(np.full(256, 2.0 ** j, np.float32))
    t = bf16_to_f64(oracle.wrmsnorm_bf16(x, w))
    assert np.array_equal(t, bf16_to_f64(oracle.rmsnorm_bf16(x)) * 2.0 ** j)


def test_wrmsnorm_weights_act_per_column_and_not_on_the_scale():
    # a one-hot weight keeps one column and zeroes the rest, while the norm
    # factor still comes from the whole row (the weight is not in the mean square)
    rng = np.random.default_rng(23)
    x = synth.f32_to_bf16_bits(rng.standard_normal((2, 384)).astype(np.float32))
    w = np.zeros(384, np.float32)
    w[77] = 1.0
    t = oracle.wrmsnorm_bf16(x, synth.f32_to_bf16_bits(w))
    ref = oracle.rmsnorm_bf16(x)
    assert np.array_equal(t[:, 77], ref[:, 77])
    assert not np.any(bf16_to_f64(np.delete(t, 77, axis=1)))


def test_wrmsnorm_close_to_float64_definition_and_amax_identity():
    rng = np.random.default_rng(24)
    x = synth.f32_to_bf16_bits((rng.standard_normal((3, 1024)) * [[0.02], [1], [30]]).astype(np.float32))
    w = synth.f32_to_bf16_bits(rng.uniform(-2, 2, 1024).astype(np.float32))
    xf, wf = bf16_to_f64(x), bf16_to_f64(w)
    r = 1.0 / np.sqrt((xf ** 2).mean(axis=1, keepdims=True) + 1e-6)
    ref = xf * wf * r
    t = bf16_to_f64(oracle.wrmsnorm_bf16(x, w))
    assert np.all(np.abs(t - ref) <= 2 ** -8 * np.abs(ref) + 1e-30)
    # the largest |t| is the rounded largest |x w| times the row's factor
    # (what a producer that only knows |x w| and sum x^2 can publish)
    for m in range(3):
        a = np.max(np.abs(xf[m] * wf))
        rf = np.float32(1.0) / np.sqrt(np.float32((xf[m] ** 2).sum() / 1024) + np.float32(1e-6))
        amax_t = bf16_to_f64(np.array([f64_to_bf16_bits_via_f32(np.float32(a) * rf)]))[0]
        assert np.max(np.abs(t[m])) == amax_t


def test_swiglu_closed_forms():
    import math
    g = _bf16([[0.0, 1.0, -1.0, 48.0, -100.0, 2.0, 1.0]])
    u = _bf16([[5.0, 1.0, 1.0, 0.75, 1.0, 0.0, -3.0]])
    h = oracle.swiglu_bf16(g, u)[0]
    assert h[0] in (0x0000, 0x8000)                      # silu(0) = 0
    assert h[1] == 0x3F3B                                 # 1/(1+e^-1) = 0.7310... -> 0.73046875
    assert bf16_to_f64(h[2:3])[0] == pytest.approx(-1 / (1 + math.e), rel=2 ** -8)
    assert bf16_to_f64(h[3:4])[0] == 36.0                 # sigmoid(48) = 1 - 1.4e-21: exactly 48 * 0.75
    assert h[4] in (0x0000, 0x8000)                       # -100 e^-100 is below every bf16
    assert bf16_to_f64(h[5:6])[0] == 0.0                  # u = 0
    s1 = 1 / (1 + math.exp(-1.0))
    assert bf16_to_f64(h[6:7])[0] == pytest.approx(-3 * s1, rel=2 ** -8)


def test_swiglu_reflection_identity():
    # silu(g) - silu(-g) = g, so h(g, u) - h(-g, u) = g u up to the two roundings
    rng = np.random.default_rng(25)
    g = synth.f32_to_bf16_bits(rng.uniform(-6, 6, 512).astype(np.float32))
    u = synth.f32_to_bf16_bits(rng.standard_normal(512).astype(np.float32))
    gf, uf = bf16_to_f64(g), bf16_to_f64(u)
    ng = synth.f32_to_bf16_bits(-gf.astype(np.float32))
    d = bf16_to_f64(oracle.swiglu_bf16(g, u)) - bf16_to_f64(oracle.swiglu_bf16(ng, u))
    bound = 2 ** -8 * (np.abs(gf * uf) + np.abs(gf * uf) / (1 + np.exp(-np.abs(gf)))) + 1e-30
    assert np.all(np.abs(d - gf * uf) <= bound)


# ---------------------------------------------------------------- decode-step walk wiring

def test_layer_sequence_wiring_with_permutation_weights():
    """Each op gets a permutation matrix (code 1) with unit scales, so an op
    copies a permuted, quantised copy of its input.  The walk's output must then
    be the input pushed through the composition of the permutations in the
    walk's dataflow order; a wrong buffer or op order gives another permutation."""
    rng = np.random.default_rng(12)
    H, I, KV = 256, 384, 128
    shapes = lambda: [("q", H, H), ("k", H, KV), ("v", H, KV), ("o", H, H),
                      ("gate", H, I), ("up", H, I), ("down", I, H)]
    ops, widths = synth.layer_program(shapes, 2)
    perms = {}
    mats = {}
    for o in ops:
        K, N = o["K"], o["N"]
        pi = rng.permutation(max(K, N))
        src = np.array([p for p in pi if p < K][:N]) if N <= K else None
        if src is None:
            src = rng.integers(0, K, size=N)
        codes = np.zeros((N, K), np.int64)
        codes[np.arange(N), src] = 1
        perms[o["matrix"]] = src
        mats[o["matrix"]] = (pack_w4(codes), np.ones((N, K // 128), np.float16))
    M = 2
    x0 = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.0, size=(M, H)).astype(np.float32) *
                                rng.choice([-1, 1], size=(M, H)).astype(np.float32))
    bufs = {i: np.zeros((M, w), np.uint16) for i, w in enumerate(widths)}
    bufs[0] = x0.copy()
    out = oracle.layer_sequence(4, ops, bufs, lambda i: mats[i])
    # Expected, approximately: follow the permutations through the dataflow.
    cur = bf16_to_f64(x0)
    for layer in range(2):
        sub = [o for o in ops if o["name"].startswith(f"L{layer}.")]
        by = {o["name"].split(".")[1]: o for o in sub}
        xn = cur / np.sqrt((cur ** 2).mean(axis=1, keepdims=True) + 1e-6)
        qv = xn[:, perms[by["q"]["matrix"]]]
        ov = qv[:, perms[by["o"]["matrix"]]]
        gv = ov[:, perms[by["gate"]["matrix"]]]
        cur = gv[:, perms[by["down"]["matrix"]]]
    got = bf16_to_f64(out[7])
    # Quantisation (step amax/127) and bf16 roundings stay well inside 0.05 of unit values.
    assert np.max(np.abs(got - cur)) < 0.05 * np.max(np.abs(cur))
    # Wrong wiring (e.g. down reading "up" instead of "gate") would break the match.
    wrong = ov[:, perms[by["up"]["matrix"]]][:, perms[by["down"]["matrix"]]]
    assert np.max(np.abs(got - wrong)) > 0.5
