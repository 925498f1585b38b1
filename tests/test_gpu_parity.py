"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: quantised activations, their scales, packed/unpacked bytes and int32
group sums are bit-exact; bf16 outputs agree within 1e-3 absolute + 1e-2
relative.  Inputs are seeded and synthetic (see synth/).
"""
import numpy as np
import pytest

import memory_bound_quantised_amd as mbq
import oracle
import synth
from tests.gpu_util import (assert_close_bf16, dev, host, oracle_rows, packed_on_device,
                            sample_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mbq.lib()
    yield
    torch.cuda.synchronize()


def special_rows(K):
    """Rows that exercise quantisation corner cases."""
    rows = []
    z = np.zeros(K, np.float32)
    rows.append(z)                                            # all zero
    t = np.zeros(K, np.float32)
    t[:8] = [127.0, 2.5, -2.5, 0.5, 1.5, -0.5, 126.5, -127.0]  # exact ties at s = 1
    rows.append(t)
    one = np.zeros(K, np.float32)
    one[K - 1] = -3.0                                         # single nonzero at the tail
    rows.append(one)
    big = np.random.default_rng(K).standard_normal(K).astype(np.float32) * 1e4
    rows.append(big)
    # scale below 127 / FLT_MAX: 1 / s overflows, so codes need the exact
    # quotient (half the columns zero, whose codes must stay 0)
    tiny = np.random.default_rng(K + 1).uniform(-3e-37, 3e-37, K).astype(np.float32)
    tiny[::2] = 0.0
    rows.append(tiny)
    return synth.f32_to_bf16_bits(np.stack(rows))


# ---------------------------------------------------------------- activation quantisation

@pytest.mark.parametrize("rmsnorm", [False, True])
@pytest.mark.parametrize("K", [128, 4096, 5120, 17408])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
def test_quantize_bit_exact(M, K, rmsnorm):
    x = synth.activations(M, K, seed=K + M)
    q, s = mbq.quantize_act(dev(x), rmsnorm=rmsnorm)
    qo, so = oracle.prologue_quant(x, oracle.PRO_RMSNORM_QUANT if rmsnorm else oracle.PRO_QUANT)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("K", [128, 4096, 17408])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_wrmsnorm_quantize_bit_exact(M, K):
    x = synth.activations(M, K, seed=K + 7 * M)
    w = synth.norm_weights(K, seed=K)
    q, s = mbq.quantize_act(dev(x), norm_w=dev(w))
    qo, so = oracle.prologue_quant(x, oracle.PRO_WRMSNORM_QUANT, norm_w=w)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("K", [128, 4096, 17408])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_swiglu_quantize(M, K):
    """The gated values match the fp64 definition within one bf16 step, and the
    codes and scales are exactly those of quantising the kernel's own gated values."""
    import torch
    g = synth.activations(M, K, seed=K + 11 * M)
    rng = np.random.default_rng(K + M)
    u = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) * 2).astype(np.float32))
    h = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    q, s = mbq.quantize_act(dev(g), up=dev(u), h_out=h)
    hg = host(h)
    ho = oracle.swiglu_bf16(g, u)
    def steps(b):   # bf16 patterns -> integers ordered like the values (+0 and -0 equal)
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    d = np.abs(steps(hg) - steps(ho))
    assert d.max() <= 1, f"{int((d > 0).sum())} differ, max {d.max()} bf16 steps"
    qo, so = oracle.quantize_act(hg)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("rmsnorm", [False, True])
@pytest.mark.parametrize("K", [128, 4096])
def test_quantize_special_rows(K, rmsnorm):
    x = special_rows(K)
    for start in range(0, len(x), 4):
        xb = x[start:start + 4]
        q, s = mbq.quantize_act(dev(xb), rmsnorm=rmsnorm)
        qo, so = oracle.prologue_quant(xb, oracle.PRO_RMSNORM_QUANT if rmsnorm else oracle.PRO_QUANT)
        assert np.array_equal(host(q), qo)
        assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))


# ---------------------------------------------------------------- layout

@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("N,K", [(1, 128), (63, 256), (65, 1152), (200, 4096)])
def test_pack_unpack_roundtrip(bits, N, K):
    canon, S = synth.weights(bits, N, K, seed=N * 7 + K)
    packed = packed_on_device(bits, canon, S, N, K)
    assert packed.numel() == mbq.packed_bytes(bits, N, K)
    c2, s2 = mbq.unpack_weights(bits, packed, N, K)
    assert np.array_equal(host(c2), canon)
    assert np.array_equal(host(s2).view(np.uint16), S.view(np.uint16))


@pytest.mark.parametrize("bits,N,K", [(4, 64, 128), (4, 1, 128), (4, 200, 384), (6, 130, 256), (6, 63, 1152),
                                      (4, 4096, 4096), (6, 1000, 1024), (4, 17408, 5120), (4, 5120, 17408),
                                      (6, 5120, 17408), (6, 17408, 5120)])
def test_pack_inplace_matches_pack(bits, N, K):
    """The in-place re-layout leaves exactly the bytes of the out-of-place pack."""
    import torch
    canon, S = synth.weights(bits, N, K, seed=N + 3 * K + bits)
    ref = packed_on_device(bits, canon, S, N, K)
    total = mbq.packed_bytes(bits, N, K)
    blob = np.concatenate([canon.reshape(-1), S.reshape(-1).view(np.uint8)])
    buf = torch.full((total,), 0x5A, dtype=torch.uint8, device="cuda")   # garbage past the canonical data
    buf[:blob.size].copy_(dev(blob))
    mbq.pack_weights_inplace(bits, buf, N, K)
    assert torch.equal(buf, ref)


@pytest.mark.parametrize("bits", [4, 6])
def test_pack_pads_rows_with_zeros(bits):
    N, K = 70, 256
    canon, S = synth.weights(bits, N, K, seed=3)
    packed = host(packed_on_device(bits, canon, S, N, K))
    tile = 4224 if bits == 4 else 6272
    G = K // 128
    # row block 1 holds rows 64..127; its local rows 6..63 are padding.  Lane l
    # of slab j holds local row 4*(l % 16) + j (W4), or in dword c of the
    # lane's 16 bytes, triple q = (4j + c) // 3, row 4*(l % 16) + q // 2 (W6).
    lanes = np.arange(64)
    for g in range(G):
        t = packed[(1 * G + g) * tile:(1 * G + g + 1) * tile]
        slabs = t[:tile - 128].reshape(-1, 64, 4, 4)      # [slab][lane][dword][byte]
        for j in range(slabs.shape[0]):
            for c in range(4):
                row = 4 * (lanes % 16) + (j if bits == 4 else ((4 * j + c) // 3) // 2)
                pad = row >= 6
                assert not slabs[j, pad, c, :].any()
                assert slabs[j, ~pad, c, :].any()
        assert not t[tile - 128:].reshape(64, 2)[6:].any()


# ---------------------------------------------------------------- exact integer sums
#
# mbq_linear_group_acc runs the product's own tile functions: FORM_MFMA is the
# whole-tile matrix-core code of the per-op linear's split and row-block forms
# and of the walk (every M), FORM_ROWSET the row-set form's (each set of 16
# rows loaded, unpacked and multiplied on its own), FORM_DOT4 the v_dot4 tile.
# Each must give the exact integer sums.

FORMS = [mbq.FORM_DOT4, mbq.FORM_MFMA, mbq.FORM_ROWSET]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", [(64, 128), (200, 1152)])
def test_group_acc_bit_exact(bits, M, N, K, form):
    canon, S = synth.weights(bits, N, K, seed=11 + N)
    x = synth.activations(M, K, seed=5)
    q, _ = oracle.quantize_act(x)
    acc = mbq.linear_group_acc(bits, dev(q), packed_on_device(bits, canon, S, N, K), N, form=form)
    assert np.array_equal(host(acc), oracle.group_acc(bits, q, canon))


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("N,K", [(5120, 17408), (17408, 5120), (16384, 5120)])
def test_group_acc_bit_exact_full_27b_shapes(bits, M, N, K, form):
    """The 27B-shaped matrices at full size: every group sum of every row."""
    canon, S = synth.weights(bits, N, K, seed=N + K + bits)
    x = synth.activations(M, K, seed=17 + M)
    q, _ = oracle.quantize_act(x)
    acc = mbq.linear_group_acc(bits, dev(q), packed_on_device(bits, canon, S, N, K), N, form=form)
    assert np.array_equal(host(acc), oracle.group_acc(bits, q, canon))


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("lo_code,q_val", [(True, -127), (True, 127), (False, 127), (False, -127)])
def test_group_acc_extreme_codes(bits, form, lo_code, q_val):
    # every weight at the most negative (or most positive) code and every
    # activation at +-127: the largest group sums the format allows
    # (|sum| up to 130048 for W4, 520192 for W6), with both signs
    N, K, M = 64, 256, 8
    code = (-8 if bits == 4 else -32) if lo_code else (7 if bits == 4 else 31)
    from tests.codes import pack
    canon = pack(bits, np.full((N, K), code))
    S = np.ones((N, K // 128), np.float16)
    q = np.full((M, K), q_val, np.int8)
    acc = host(mbq.linear_group_acc(bits, dev(q), packed_on_device(bits, canon, S, N, K), N, form=form))
    assert np.all(acc == 128 * q_val * code)
    assert np.array_equal(acc, oracle.group_acc(bits, q, canon))


# ---------------------------------------------------------------- the linear

@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
# the row-block form (the first four) and the split form (a few row blocks over
# many k groups; more than 512 row blocks)
@pytest.mark.parametrize("N,K", [(1, 128), (200, 1152), (1000, 4096), (4096, 4096), (1000, 8192), (200, 17408),
                                 (33000, 256)])
def test_linear_vs_oracle(bits, M, N, K):
    canon, S = synth.weights(bits, N, K, seed=1)
    x = synth.activations(M, K)
    q, s = oracle.quantize_act(x)
    y = mbq.linear(bits, dev(q), dev(s), packed_on_device(bits, canon, S, N, K), N)
    assert_close_bf16(host(y), oracle.linear(bits, q, s, canon, S), f"W{bits} M={M} {N}x{K}")


# The forms without partials: their edges.  Row-set form (four workgroups per
# row block, at most 64 blocks): 3070 x 4224, 48 blocks, the last one 62 rows,
# 33 groups over 16 waves (uneven ranges); 3100 x 8192, 64 groups (ranges past
# the all-at-once count, so through the batched loop).  Row-block form:
# 16384 x 128, 256 blocks of one group (most waves idle); 8190 x 4096, 128
# blocks, the last one 62 rows, 32 groups over 16 (W4) or 8 (W6) waves;
# 4200 x 8320, 66 blocks, 65 groups over 4 waves (batched, uneven).
@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [1, 3, 4, 8])
@pytest.mark.parametrize("N,K", [(3070, 4224), (3100, 8192), (16384, 128), (8190, 4096), (4200, 8320)])
def test_linear_row_block_form_vs_oracle(bits, M, N, K):
    canon, S = synth.weights(bits, N, K, seed=N ^ K)
    x = synth.activations(M, K)
    q, s = oracle.quantize_act(x)
    y = mbq.linear(bits, dev(q), dev(s), packed_on_device(bits, canon, S, N, K), N)
    assert_close_bf16(host(y), oracle.linear(bits, q, s, canon, S), f"W{bits} M={M} {N}x{K}")


# The linear with its prologue and quantisation inside it: bitwise the
# quantisation call followed by the linear (every prologue; 4096 x 4096,
# 3070 x 4224 and 1024 x 5120 take the row-set form, 5120 x 8192,
# 5120 x 17408 and 4096 x 20480 the row-block form with 4 waves and batched
# ranges).
@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("prologue", [0, 1, 2, 3])
@pytest.mark.parametrize("M", [1, 3, 8])
# fused (M x K codes in LDS) except 4096 x 20480 at M = 8 (more codes than the
# LDS holds: the prologue kernel first) and 1000 x 8192 (the split form)
@pytest.mark.parametrize("N,K", [(4096, 4096), (3070, 4224), (5120, 8192), (1024, 5120), (5120, 17408),
                                 (4096, 20480), (1000, 8192)])
def test_linear_prologue_matches_quantise_then_linear(bits, prologue, M, N, K):
    canon, S = synth.weights(bits, N, K, seed=N + K + prologue)
    packed = packed_on_device(bits, canon, S, N, K)
    x = dev(synth.activations(M, K))
    up = dev(synth.activations(M, K, seed=77)) if prologue == mbq.PRO_SWIGLU_QUANT else None
    nw = dev(synth.norm_weights(K, 5)) if prologue == mbq.PRO_WRMSNORM_QUANT else None
    y = host(mbq.linear_prologue(bits, x, packed, N, prologue, up=up, norm_w=nw))
    q, s = mbq.quantize_act(x, rmsnorm=prologue == mbq.PRO_RMSNORM_QUANT, norm_w=nw, up=up)
    ref = host(mbq.linear(bits, q, s, packed, N))
    assert np.array_equal(y, ref), f"W{bits} prologue {prologue} M={M} {N}x{K}"


@pytest.mark.parametrize("prologue", [0, 1])
def test_linear_prologue_vs_oracle(prologue):
    N, K, M = 4096, 4096, 3
    canon, S = synth.weights(4, N, K, seed=21)
    x = synth.activations(M, K)
    y = host(mbq.linear_prologue(4, dev(x), packed_on_device(4, canon, S, N, K), N, prologue))
    assert_close_bf16(y, oracle.op(4, x, prologue, canon, S), f"prologue {prologue}")


# Full-size shapes of the 9B- and 27B-shaped decode steps; outputs checked on sampled rows.
FULL_SHAPES = [(4096, 4096), (1024, 4096), (12288, 4096), (4096, 12288), (16384, 5120),
               (1024, 5120), (5120, 8192), (17408, 5120), (5120, 17408)]


@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("N,K", FULL_SHAPES)
def test_linear_full_size_sampled(bits, M, N, K):
    canon, S = synth.weights(bits, N, K, seed=N + K)
    x = synth.activations(M, K)
    q, s = oracle.quantize_act(x)
    y = host(mbq.linear(bits, dev(q), dev(s), packed_on_device(bits, canon, S, N, K), N))
    rows = sample_rows(np.random.default_rng(N), N)
    ref = oracle.linear(bits, q, s, canon[rows], S[rows])
    assert_close_bf16(y[:, rows], ref, f"W{bits} M={M} {N}x{K}")


# Row m of an M-row call is bitwise the one-row call, in every form: the
# row-set form (3000 x 5120: 47 row blocks), the row-block form with 16 (W4)
# or 8 (W6) waves (8192 x 1024) and with 4 (8192 x 8192), and the split form
# (1000 x 8192).
@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [3, 4, 8])
@pytest.mark.parametrize("N,K", [(3000, 5120), (8192, 1024), (8192, 8192), (1000, 8192)])
def test_linear_rows_independent_and_deterministic(bits, M, N, K):
    canon, S = synth.weights(bits, N, K, seed=9)
    packed = packed_on_device(bits, canon, S, N, K)
    x = synth.activations(M, K)
    q, s = oracle.quantize_act(x)
    y = host(mbq.linear(bits, dev(q), dev(s), packed, N))
    yb = host(mbq.linear(bits, dev(q), dev(s), packed, N))
    assert np.array_equal(y, yb)
    for m in range(M):
        ym = host(mbq.linear(bits, dev(q[m:m + 1]), dev(s[m:m + 1]), packed, N))
        assert np.array_equal(ym, y[m:m + 1]), f"W{bits} {N}x{K} row {m} of {M}"



def test_linear_zero_row():
    N, K = 256, 1024
    canon, S = synth.weights(4, N, K, seed=2)
    x = synth.activations(2, K)
    x[0] = 0
    q, s = oracle.quantize_act(x)
    y = host(mbq.linear(4, dev(q), dev(s), packed_on_device(4, canon, S, N, K), N))
    assert not y[0].any()


def test_linear_workspace_reused_across_shapes():
    """The split counters reset themselves, so one workspace serves any later call."""
    import torch
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device="cuda")
    for (bits, M, N, K) in [(4, 1, 4096, 4096), (6, 4, 200, 1152), (4, 3, 17408, 5120), (4, 1, 64, 128),
                            (6, 2, 5120, 17408)]:
        canon, S = synth.weights(bits, N, K, seed=M * N)
        x = synth.activations(M, K)
        q, s = oracle.quantize_act(x)
        y = host(mbq.linear(bits, dev(q), dev(s), packed_on_device(bits, canon, S, N, K), N, ws=ws))
        rows = sample_rows(np.random.default_rng(1), N)
        assert_close_bf16(y[:, rows], oracle.linear(bits, q, s, canon[rows], S[rows]), f"{bits} {N}x{K}")
    torch.cuda.synchronize()
    assert not ws[:65536].any()   # counters region left at zero


# ---------------------------------------------------------------- decode-step walk

def _run_sequence(bits, shapes_fn, n_layers, M, distinct, seed_base=0, fused=True, runs=1, dataflow="plain",
                  x0=None):
    import torch
    ops, widths = synth.layer_program(shapes_fn, n_layers, distinct_buffers=distinct, dataflow=dataflow)
    mats = {}
    norms = {}   # one device copy per set of norm weights: ops sharing a norm share its pointer
    dev_ops = []
    for o in ops:
        canon, S = synth.weights(bits, o["N"], o["K"], seed=1 + o["matrix"] + seed_base)
        mats[o["matrix"]] = (canon, S)
        d = dict(bits=bits, prologue=o["prologue"], N=o["N"], K=o["K"],
                 packed=packed_on_device(bits, canon, S, o["N"], o["K"]),
                 in_buf=o["in_buf"], out_buf=o["out_buf"])
        if "norm_seed" in o:
            o["norm_w"] = synth.norm_weights(o["K"], o["norm_seed"])
            if o["norm_seed"] not in norms:
                norms[o["norm_seed"]] = dev(o["norm_w"])
            d["norm_w"] = norms[o["norm_seed"]]
        if "in_buf2" in o:
            d["in_buf2"] = o["in_buf2"]
        dev_ops.append(d)
    bufs = [torch.zeros((M, w), dtype=torch.bfloat16, device="cuda") for w in widths]
    if x0 is None:
        x0 = synth.activations(M, widths[0])
    bufs[0].copy_(dev(x0))
    seq = mbq.LayerSequence(dev_ops, bufs, M, fused=fused)
    outs = []
    for _ in range(runs):
        bufs[0].copy_(dev(x0))
        seq.run()
        if fused:
            seq.check()
        torch.cuda.synchronize()
        outs.append([host(b) for b in bufs])
    if runs > 1:
        return ops, mats, outs, x0
    return ops, mats, outs[0], x0


def _small_shapes():
    H, I, KV = 256, 384, 128
    return [("q", H, H), ("k", H, KV), ("v", H, KV), ("o", H, H),
            ("gate", H, I), ("up", H, I), ("down", I, H)]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_layer_sequence_teacher_forced_small(bits, M, fused):
    ops, mats, bufs, _ = _run_sequence(bits, _small_shapes, 3, M, distinct=True, fused=fused)
    for o in ops:
        x = np.ascontiguousarray(bufs[o["in_buf"]][:, :o["K"]])
        ref = oracle.op(bits, x, o["prologue"], *mats[o["matrix"]])
        assert_close_bf16(bufs[o["out_buf"]], ref, o["name"])


def _bf16_steps(b):
    """bf16 bit patterns -> integers ordered like the values (+0 and -0 equal)."""
    b = b.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _gpu_swiglu(g_bits, u_bits):
    """The gated values h = bf16(silu(g) * u) as the GPU computes them (fp32, the
    library's expf), from the per-op SwiGLU quantisation kernel, which runs the
    same device function on the same bytes as the walk's gate/up finalisers."""
    import torch
    h = torch.zeros(g_bits.shape, dtype=torch.bfloat16, device="cuda")
    mbq.quantize_act(dev(g_bits), up=dev(u_bits), h_out=h)
    return host(h)


def _oracle_op_rows(bits, bufs, o, mats, rows=None):
    """Oracle outputs of op o from the walk's own input buffers (teacher forced).

    A SwiGLU op is teacher-forced at its gated input: the GPU evaluates silu in
    fp32 and the oracle in fp64, so h may differ by one bf16 step, and a code
    flipped by that step moves an output with heavy cancellation by more than
    the linear's tolerance.  The oracle therefore quantises the GPU's h (pinned
    here to the fp64 definition within one bf16 step) and runs the linear on
    it; the quantisation of a given h is bit-exact on both sides."""
    x = np.ascontiguousarray(bufs[o["in_buf"]][:, :o["K"]])
    canon, S = mats[o["matrix"]]
    if rows is not None:
        canon, S = canon[rows], S[rows]
    if o["prologue"] == oracle.PRO_SWIGLU_QUANT:
        u = np.ascontiguousarray(bufs[o["in_buf2"]][:, :o["K"]])
        h = _gpu_swiglu(x, u)
        d = np.abs(_bf16_steps(h) - _bf16_steps(oracle.swiglu_bf16(x, u)))
        assert d.max() <= 1, f"{o['name']}: gated input {int(d.max())} bf16 steps from the fp64 definition"
        return oracle.op(bits, h, oracle.PRO_QUANT, canon, S)
    return oracle.op(bits, x, o["prologue"], canon, S, o.get("norm_w"), None)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("bits", [4, 6])
def test_sequence_quantises_corner_rows(bits, fused):
    """The walk's input quantisation on the corner-case rows (all zero, exact
    ties, a lone value at the tail, large values, a scale whose reciprocal
    overflows), then an op on its output.  Outputs are compared row by row
    relative to the row's largest output, since the tiny row's outputs sit far
    below the absolute tolerance."""
    import torch
    K, N = 384, 256
    x = special_rows(K)
    M = len(x)
    ops = [dict(name="a", K=K, N=N, in_buf=0, out_buf=1, prologue=oracle.PRO_QUANT),
           dict(name="b", K=N, N=128, in_buf=1, out_buf=2, prologue=oracle.PRO_QUANT)]
    mats, dev_ops = {}, []
    for i, o in enumerate(ops):
        o["matrix"] = i
        mats[i] = synth.weights(bits, o["N"], o["K"], seed=700 + i)
        dev_ops.append(dict(bits=bits, prologue=o["prologue"], N=o["N"], K=o["K"], in_buf=o["in_buf"],
                            out_buf=o["out_buf"], packed=packed_on_device(bits, *mats[i], o["N"], o["K"])))
    bufs = [torch.zeros((M, w), dtype=torch.bfloat16, device="cuda") for w in (K, N, 128)]
    bufs[0].copy_(dev(x))
    seq = mbq.LayerSequence(dev_ops, bufs, M, fused=fused)
    seq.run()
    if fused:
        seq.check()
    torch.cuda.synchronize()
    hb = [host(b) for b in bufs]
    for o in ops:
        y = synth.bf16_bits_to_f32(hb[o["out_buf"]]).astype(np.float64)
        ref = synth.bf16_bits_to_f32(_oracle_op_rows(bits, hb, o, mats)).astype(np.float64)
        for m in range(M):
            top = np.abs(ref[m]).max()
            if top == 0.0:
                assert np.all(y[m] == 0.0), f"{o['name']} row {m}"
                continue
            err = np.abs(y[m] - ref[m]) / top
            assert np.all(err <= 1e-3 + 1e-2 * np.abs(ref[m]) / top), f"{o['name']} row {m}: max {err.max()}"


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_layer_sequence_swiglu_dataflow_small(bits, M, fused):
    """The walk with weighted RMSNorms and the SwiGLU gate in front of down."""
    ops, mats, bufs, _ = _run_sequence(bits, _small_shapes, 3, M, distinct=True, fused=fused,
                                       dataflow="swiglu")
    for o in ops:
        assert_close_bf16(bufs[o["out_buf"]], _oracle_op_rows(bits, bufs, o, mats), o["name"])


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("M", [1, 3])
def test_layer_sequence_swiglu_dataflow_9b_layers(M, fused):
    ops, mats, bufs, _ = _run_sequence(4, synth.layer_shapes_9b, 2, M, distinct=True, fused=fused,
                                       dataflow="swiglu")
    rng = np.random.default_rng(7)
    for o in ops:
        rows = sample_rows(rng, o["N"], 128)
        assert_close_bf16(bufs[o["out_buf"]][:, rows], _oracle_op_rows(4, bufs, o, mats, rows), o["name"])


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [1, 8])
def test_sequence_gate_and_norm_inputs_from_before_the_walk(bits, M, fused):
    """A SwiGLU op whose gate and up are written before the walk (the fused
    walk gates them in its kernel-start pass), a weighted-RMSNorm op on its
    output, and one on an input from before the walk."""
    import torch
    widths = [384, 384, 256, 256, 128, 256]
    w1, w2 = synth.norm_weights(256, 11), synth.norm_weights(256, 12)
    ops = [dict(name="down", K=384, N=256, in_buf=0, in_buf2=1, out_buf=2, prologue=oracle.PRO_SWIGLU_QUANT),
           dict(name="a", K=256, N=128, in_buf=2, out_buf=4, prologue=oracle.PRO_WRMSNORM_QUANT, norm_w=w1),
           dict(name="b", K=256, N=256, in_buf=3, out_buf=5, prologue=oracle.PRO_WRMSNORM_QUANT, norm_w=w2)]
    mats, dev_ops = {}, []
    for i, o in enumerate(ops):
        o["matrix"] = i
        mats[i] = synth.weights(bits, o["N"], o["K"], seed=300 + i)
        d = dict(bits=bits, prologue=o["prologue"], N=o["N"], K=o["K"], in_buf=o["in_buf"], out_buf=o["out_buf"],
                 packed=packed_on_device(bits, *mats[i], o["N"], o["K"]))
        if "in_buf2" in o:
            d["in_buf2"] = o["in_buf2"]
        if "norm_w" in o:
            d["norm_w"] = dev(o["norm_w"])
        dev_ops.append(d)
    bufs = [torch.zeros((M, w), dtype=torch.bfloat16, device="cuda") for w in widths]
    for b, seed in ((0, 21), (1, 22), (3, 23)):
        bufs[b].copy_(dev(synth.activations(M, widths[b], seed=seed)))
    seq = mbq.LayerSequence(dev_ops, bufs, M, fused=fused)
    for _ in range(2):   # the second run sees the first one's tags in the workspace
        seq.run()
        if fused:
            seq.check()
        torch.cuda.synchronize()
        hb = [host(b) for b in bufs]
        for o in ops:
            assert_close_bf16(hb[o["out_buf"]], _oracle_op_rows(bits, hb, o, mats), o["name"])


@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_layer_sequence_9b_layers_teacher_forced(bits, M):
    ops, mats, bufs, _ = _run_sequence(bits, synth.layer_shapes_9b, 2, M, distinct=True)
    rng = np.random.default_rng(4)
    for o in ops:
        x = np.ascontiguousarray(bufs[o["in_buf"]][:, :o["K"]])
        canon, S = mats[o["matrix"]]
        rows = sample_rows(rng, o["N"], 128)
        ref = oracle_rows(bits, x, o["prologue"], canon, S, rows)
        assert_close_bf16(bufs[o["out_buf"]][:, rows], ref, o["name"])


@pytest.mark.parametrize("bits,M", [(4, 1), (4, 2), (4, 3), (4, 4), (4, 5), (4, 6), (4, 7), (4, 8),
                                    (6, 1), (6, 2), (6, 3), (6, 4), (6, 5), (6, 6), (6, 7), (6, 8)])
def test_layer_sequence_27b_layer_teacher_forced(bits, M):
    """One 27B-shaped layer at every row count, both bit widths: q is 16384
    wide and o reads its first 8192 columns."""
    ops, mats, bufs, _ = _run_sequence(bits, synth.layer_shapes_27b, 1, M, distinct=True)
    rng = np.random.default_rng(5)
    for o in ops:
        x = np.ascontiguousarray(bufs[o["in_buf"]][:, :o["K"]])
        canon, S = mats[o["matrix"]]
        rows = sample_rows(rng, o["N"], 128)
        ref = oracle_rows(bits, x, o["prologue"], canon, S, rows)
        assert_close_bf16(bufs[o["out_buf"]][:, rows], ref, o["name"])


@pytest.mark.parametrize("bits,M", [(4, 1), (4, 2), (4, 3), (4, 4), (4, 6), (4, 8), (6, 1), (6, 3), (6, 4), (6, 8)])
def test_layer_sequence_27b_layer_swiglu_dataflow(bits, M):
    """The same layer through the walk's other kernel form: weighted RMSNorms in
    front of q/k/v and gate/up, the SwiGLU gate in front of down.  From M = 3 on
    a finalising workgroup's waves share each gate/up pair's gather, and a
    share can end exactly where the gate's contributions end and the up's
    begin (equal counts): that share holds gate sums only."""
    ops, mats, bufs, _ = _run_sequence(bits, synth.layer_shapes_27b, 1, M, distinct=True, dataflow="swiglu")
    rng = np.random.default_rng(8)
    for o in ops:
        rows = sample_rows(rng, o["N"], 128)
        assert_close_bf16(bufs[o["out_buf"]][:, rows], _oracle_op_rows(bits, bufs, o, mats, rows), o["name"])


@pytest.mark.parametrize("bits", [4, 6])
def test_layer_sequence_fused_deterministic_and_rerunnable(bits):
    """Two runs of one prepared walk give bitwise equal buffers, and the fused
    walk agrees with the unfused one within the output tolerance."""
    ops, mats, outs, _ = _run_sequence(bits, _small_shapes, 4, 3, distinct=True, runs=2)
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
    _, _, unf, _ = _run_sequence(bits, _small_shapes, 4, 3, distinct=True, fused=False)
    # first layer: same inputs, so outputs agree within the linear's tolerance
    for o in ops[:7]:
        assert_close_bf16(outs[0][o["out_buf"]], unf[o["out_buf"]], o["name"])


@pytest.mark.parametrize("dataflow", ["plain", "swiglu"])
def test_layer_sequence_graph_replays(dataflow):
    """The fused walk captured in a HIP graph: each replay, on an input written
    between replays (every other buffer zeroed), equals an eager run on that
    input bit for bit.  Every launch tags its hand-over words with the
    workspace's next epoch, read and advanced on the device, so a replay never
    takes a word the previous one left."""
    import torch
    M = 2
    ops, widths = synth.layer_program(_small_shapes, 3, distinct_buffers=True, dataflow=dataflow)
    norms, dev_ops = {}, []
    for o in ops:
        canon, S = synth.weights(4, o["N"], o["K"], seed=300 + o["matrix"])
        d = dict(bits=4, prologue=o["prologue"], N=o["N"], K=o["K"], packed=packed_on_device(4, canon, S, o["N"], o["K"]),
                 in_buf=o["in_buf"], out_buf=o["out_buf"])
        if "norm_seed" in o:
            if o["norm_seed"] not in norms:
                norms[o["norm_seed"]] = dev(synth.norm_weights(o["K"], o["norm_seed"]))
            d["norm_w"] = norms[o["norm_seed"]]
        if "in_buf2" in o:
            d["in_buf2"] = o["in_buf2"]
        dev_ops.append(d)
    bufs = [torch.zeros((M, w), dtype=torch.bfloat16, device="cuda") for w in widths]
    seq = mbq.LayerSequence(dev_ops, bufs, M, fused=True)
    inputs = [dev(synth.activations(M, widths[0], seed=500 + i)) for i in range(3)]

    def load(i):
        for b in bufs[1:]:
            b.zero_()
        bufs[0].copy_(inputs[i])

    eager = []
    for i in range(3):
        load(i)
        seq.run()
        seq.check()
        eager.append([host(b) for b in bufs])
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        seq.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    try:
        with torch.cuda.graph(g):
            seq.run()
    except RuntimeError as e:   # pragma: no cover - depends on the runtime
        pytest.skip(f"the runtime does not capture the walk's cooperative launch: {e}")
    for i in (2, 0, 1, 2, 0):
        load(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        seq.check()
        for k, (a, b) in enumerate(zip([host(b) for b in bufs], eager[i])):
            assert np.array_equal(a, b), f"replay of input {i}, buffer {k}"


@pytest.mark.parametrize("shapes,M,dataflow", [("27b", 8, "plain"), ("27b", 3, "plain"), ("9b", 4, "swiglu")])
def test_layer_sequence_shared_gathers_reproducible(shapes, M, dataflow):
    """Where a finalising workgroup's waves share a row block's gather (the o
    and down blocks of these layers, gate/up pairs in the SwiGLU walk), the
    parts are added in a fixed order: two runs agree bitwise."""
    fn = synth.layer_shapes_27b if shapes == "27b" else synth.layer_shapes_9b
    _, _, outs, _ = _run_sequence(4, fn, 1, M, distinct=True, runs=2, dataflow=dataflow)
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("shapes,layers,M,bits,dataflow", [
    ("small", 3, 3, 4, "plain"), ("small", 3, 8, 6, "swiglu"), ("27b", 1, 3, 4, "plain"), ("9b", 1, 4, 6, "swiglu")])
def test_layer_sequence_batch_invariant(shapes, layers, M, bits, dataflow, fused):
    """Row m of an M-row walk is bitwise the walk of that row alone: every
    intermediate buffer of every layer (the verify rows cost nothing in the
    quality of what is computed for each of them)."""
    fn = {"small": _small_shapes, "27b": synth.layer_shapes_27b, "9b": synth.layer_shapes_9b}[shapes]
    _, _, outs, x0 = _run_sequence(bits, fn, layers, M, distinct=True, fused=fused, dataflow=dataflow)
    for m in range(M):
        _, _, one, _ = _run_sequence(bits, fn, layers, 1, distinct=True, fused=fused, dataflow=dataflow,
                                     x0=x0[m:m + 1])
        for i, (a, b) in enumerate(zip(outs, one)):
            assert np.array_equal(a[m:m + 1], b), f"row {m} of buffer {i}"


@pytest.mark.parametrize("M", [1, 3])
def test_layer_sequence_bench_configuration(M):
    """The 36-layer 9B-shaped walk with reused buffers, as the benchmark runs it.
    The last layer's o, gate, up and down inputs survive in their buffers and are
    checked teacher-forced on sampled rows."""
    ops, mats, bufs, _ = _run_sequence(4, synth.layer_shapes_9b, 36, M, distinct=False)
    last = [o for o in ops if o["name"].startswith("L35.") and o["name"].split(".")[1]
            in ("o", "gate", "up", "down")]
    rng = np.random.default_rng(6)
    for o in last:
        x = np.ascontiguousarray(bufs[o["in_buf"]][:, :o["K"]])
        canon, S = mats[o["matrix"]]
        rows = sample_rows(rng, o["N"], 128)
        ref = oracle_rows(4, x, o["prologue"], canon, S, rows)
        assert_close_bf16(bufs[o["out_buf"]][:, rows], ref, o["name"])
    for b in bufs:
        assert np.all(np.isfinite(synth.bf16_bits_to_f32(b)))


@pytest.mark.parametrize("bits", [4, 6])
def test_fused_and_unfused_walks_share_one_workspace(bits):
    """The fused walk, then the unfused one, then the fused one again, all on one
    workspace: the two forms use disjoint regions of it, so each run matches the
    oracle (teacher forced) and the fused plan survives the unfused run."""
    import torch
    M = 3
    ops, widths = synth.layer_program(_small_shapes, 2, distinct_buffers=True)
    mats, dev_ops = {}, []
    for o in ops:
        mats[o["matrix"]] = synth.weights(bits, o["N"], o["K"], seed=1 + o["matrix"])
        dev_ops.append(dict(bits=bits, prologue=o["prologue"], N=o["N"], K=o["K"], in_buf=o["in_buf"],
                            out_buf=o["out_buf"], packed=packed_on_device(bits, *mats[o["matrix"]], o["N"], o["K"])))
    bufs = [torch.zeros((M, w), dtype=torch.bfloat16, device="cuda") for w in widths]
    x0 = synth.activations(M, widths[0])
    fused = mbq.LayerSequence(dev_ops, bufs, M, fused=True)
    unfused = mbq.LayerSequence(dev_ops, bufs, M, fused=False, ws=fused.ws)
    for seq in (fused, unfused, fused, unfused):
        for b in bufs:
            b.zero_()
        bufs[0].copy_(dev(x0))
        seq.run()
        if seq.fused:
            seq.check()
        torch.cuda.synchronize()
        hb = [host(b) for b in bufs]
        for o in ops:
            assert_close_bf16(hb[o["out_buf"]], _oracle_op_rows(bits, hb, o, mats), o["name"])
