"""The C-ABI library loads, exports what include/mbq.h declares, and rejects bad
arguments before touching the GPU.  No compute call runs here."""
import ctypes
import os
import re

import pytest

import memory_bound_quantised_amd as mbq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mbq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(mbq.LIB_PATH),
                                reason="libmbq.so not built (python -m memory_bound_quantised_amd.build)")

A = 1 << 20          # a 256-byte-aligned fake device address; never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mbq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("mbq_quantize_act", "mbq_w4a8_linear", "mbq_w6a8_linear", "mbq_layer_sequence",
                     "mbq_pack_weights"):
        assert required in names


def test_every_declared_symbol_is_exported():
    L = ctypes.CDLL(mbq.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing
    assert sorted(mbq.EXPORTS) == declared_functions()


def test_status_strings_and_version():
    L = mbq.lib()
    assert L.mbq_status_string(0) == b"ok"
    assert b"bits" in L.mbq_status_string(-3)
    assert L.mbq_status_string(12345) == b"unknown status"
    assert L.mbq_version().startswith(b"mbq")
    assert L.mbq_last_hip_error() == 0


@pytest.mark.parametrize("bits,N,K,tile", [(4, 1, 128, 4224), (4, 64, 4096, 4224), (4, 65, 256, 4224),
                                           (6, 4096, 4096, 6272), (6, 200, 1152, 6272)])
def test_packed_bytes_formula(bits, N, K, tile):
    assert mbq.packed_bytes(bits, N, K) == ((N + 63) // 64) * (K // 128) * tile
    # never smaller than the algorithmic bytes: codes plus fp16 group scales
    assert mbq.packed_bytes(bits, N, K) >= N * K * bits // 8 + N * (K // 128) * 2


def test_packed_bytes_rejects():
    L = mbq.lib()
    assert L.mbq_packed_bytes(5, 64, 128) == -3
    assert L.mbq_packed_bytes(4, 0, 128) == -2
    assert L.mbq_packed_bytes(4, 64, 100) == -2
    assert L.mbq_packed_bytes(4, 64, 0) == -2


def test_linear_argument_validation():
    L = mbq.lib()
    ws_need = L.mbq_linear_workspace_bytes(4, 1, 4096, 4096)
    assert ws_need > 0
    f = L.mbq_w4a8_linear
    assert f(1, 4096, 4096, None, A, A, A, A, ws_need, None) == -1          # null q
    assert f(0, 4096, 4096, A, A, A, A, A, ws_need, None) == -2             # M = 0
    assert f(9, 4096, 4096, A, A, A, A, A, ws_need, None) == -2             # M = 9
    assert f(1, 4096, 4000, A, A, A, A, A, ws_need, None) == -2             # K % 128
    assert f(1, 0, 4096, A, A, A, A, A, ws_need, None) == -2                # N = 0
    assert f(1, 4096, 4096, A, A, A + 16, A, A, ws_need, None) == -4        # packed not 256-aligned
    assert f(1, 4096, 4096, A + 4, A, A, A, A, ws_need, None) == -4         # q not 16-aligned
    assert f(1, 4096, 4096, A, A, A, A, A, ws_need - 1, None) == -5         # workspace too small
    assert f(1, 4096, 4096, A, A, A, A, None, ws_need, None) == -5          # no workspace
    assert L.mbq_w6a8_linear(1, 64, 128, A, A, A, A, A + 8, 1 << 30, None) == -4   # ws alignment
    assert L.mbq_linear_workspace_bytes(7, 1, 64, 128) == -3
    assert L.mbq_linear_group_acc(5, 1, 1, 64, 128, A, A, A, None) == -3
    assert L.mbq_linear_group_acc(4, 1, 1, 64, 128, None, A, A, None) == -1
    assert L.mbq_linear_group_acc(4, 3, 1, 64, 128, A, A, A, None) == -2    # no such tile form
    assert L.mbq_linear_group_acc(4, 0, 9, 64, 128, A, A, A, None) == -2


def test_linear_noalloc_validation():
    """Argument checks of the allocation-free linear, all before any device call."""
    L = mbq.lib()
    f = L.mbq_linear_noalloc
    assert f(5, 1, 4096, 4096, A, A, A, A, None) == -3                  # bits
    assert f(4, 1, 4096, 4096, None, A, A, A, None) == -1               # null q
    assert f(4, 1, 4096, 4096, A, A, A, None, None) == -1               # null y
    assert f(4, 9, 4096, 4096, A, A, A, A, None) == -2                  # M = 9
    assert f(4, 1, 4096, 4000, A, A, A, A, None) == -2                  # K % 128
    assert f(4, 1, 4096, 4096, A, A, A + 16, A, None) == -4             # packed not 256-aligned
    # the library's array (8 MiB + 64 KiB) holds the split-K scratch of every
    # supported shape: the planner keeps row blocks x splits below 4096
    cap = (8 << 20) + (64 << 10)
    worst = 0
    for N in [1, 64, 1000, 4096, 5120, 17408, 64 * 2047, 64 * 2048, 1 << 20]:
        for K in [128, 1024, 4096, 17408, 1 << 20, 1 << 24]:
            for bits in (4, 6):
                worst = max(worst, L.mbq_linear_workspace_bytes(bits, 8, N, K))
    assert 0 < worst <= cap


def test_linear_prologue_validation():
    """Argument checks of the linear with its prologue inside, all before any device call."""
    L = mbq.lib()
    f = L.mbq_linear_prologue
    need = L.mbq_linear_prologue_workspace_bytes(4, 3, 4096, 4096)
    lin = L.mbq_linear_workspace_bytes(4, 3, 4096, 4096)
    assert need >= 3 * 4096 + 256 + lin                                          # codes, scales, linear scratch
    assert L.mbq_linear_prologue_workspace_bytes(5, 3, 4096, 4096) == -3
    assert L.mbq_linear_prologue_workspace_bytes(4, 9, 4096, 4096) == -2
    def call(bits=4, pro=0, M=3, N=4096, K=4096, x=A, u=None, w=None, packed=A, y=A, ws=A, wsb=need):
        return f(bits, pro, M, N, K, x, u, w, packed, y, ws, wsb, None)
    assert call(bits=5) == -3
    assert call(pro=4) == -6 and call(pro=-1) == -6                               # unknown prologue
    assert call(x=None) == -1 and call(y=None) == -1 and call(packed=None) == -1
    assert call(pro=3) == -1                                                      # SwiGLU without up rows
    assert call(pro=2) == -1                                                      # weighted norm without weights
    assert call(M=9) == -2 and call(K=4000) == -2
    assert call(packed=A + 16) == -4 and call(x=A + 8) == -4
    assert call(pro=3, u=A + 8) == -4 and call(pro=2, w=A + 8) == -4
    assert call(wsb=need - 1) == -5 and call(ws=None) == -5
    assert call(ws=A + 16) == -4


def test_stream_read_validation():
    L = mbq.lib()
    assert L.mbq_stream_read(None, 1024, A, None) == -1
    assert L.mbq_stream_read(A, 1024, None, None) == -1
    assert L.mbq_stream_read(A, 0, A, None) == -2
    assert L.mbq_stream_read(A, 1000, A, None) == -2          # not whole KiB
    assert L.mbq_stream_read(A + 16, 1024, A, None) == -4     # buffer not 256-aligned


def test_quant_and_pack_validation():
    L = mbq.lib()
    assert L.mbq_quantize_act(1, 4096, None, A, A, None) == -1
    assert L.mbq_quantize_act(9, 4096, A, A, A, None) == -2
    assert L.mbq_rmsnorm_quantize_act(1, 64, A, A, A, None) == -2
    assert L.mbq_quantize_act(1, 4096, A + 2, A, A, None) == -4
    assert L.mbq_pack_weights(3, 64, 128, A, A, A, None) == -3
    assert L.mbq_pack_weights(4, 64, 128, None, A, A, None) == -1
    assert L.mbq_pack_weights(4, 64, 130, A, A, A, None) == -2
    assert L.mbq_pack_weights(6, 64, 128, A, A, A + 128, None) == -4
    assert L.mbq_unpack_weights(6, 64, 128, A, A, None, None) == -1


def _program(ops):
    arr = (mbq.MbqOp * len(ops))()
    for i, o in enumerate(ops):
        arr[i] = mbq.MbqOp(*o)
    return arr


def test_sequence_program_validation():
    L = mbq.lib()
    W = (ctypes.c_int64 * 3)(256, 512, 256)
    good = _program([(4, 1, 512, 256, A, 0, 1), (4, 0, 256, 512, A, 1, 2)])
    assert L.mbq_sequence_workspace_bytes(good, 2, W, 3, 1) > 0
    bad_cases = {
        "out of range buffer": ([(4, 1, 512, 256, A, 0, 3)], -6),
        "in place": ([(4, 1, 256, 256, A, 0, 0)], -6),
        "N != width": ([(4, 1, 256, 256, A, 0, 1)], -6),
        "K > width": ([(4, 1, 512, 384, A, 0, 1)], -6),
        "bad prologue": ([(4, 7, 512, 256, A, 0, 1)], -6),
        "bad bits": ([(5, 1, 512, 256, A, 0, 1)], -3),
        "null weights": ([(4, 1, 512, 256, None, 0, 1)], -1),
        "misaligned weights": ([(4, 1, 512, 256, A + 64, 0, 1)], -4),
        "same output twice in a phase": ([(4, 1, 512, 256, A, 0, 1), (4, 1, 512, 256, A, 0, 1)], -6),
    }
    for name, (ops, want) in bad_cases.items():
        assert L.mbq_sequence_workspace_bytes(_program(ops), len(ops), W, 3, 1) == want, name
    assert L.mbq_sequence_workspace_bytes(good, 2, W, 3, 9) == -2
    assert L.mbq_sequence_workspace_bytes(good, 2, W, 3, 8) > 0
    assert L.mbq_sequence_workspace_bytes(good, 0, W, 3, 1) == -6
    W_bad = (ctypes.c_int64 * 3)(256, 500, 256)
    assert L.mbq_sequence_workspace_bytes(good, 2, W_bad, 3, 1) == -6
    bufs = (ctypes.c_void_p * 3)(A, A, A)
    need = L.mbq_sequence_workspace_bytes(good, 2, W, 3, 1)
    f = L.mbq_layer_sequence_unfused
    assert f(good, 2, bufs, W, 3, 1, A, 1, None) == -5
    assert f(good, 2, None, W, 3, 1, A, need, None) == -1
    bufs_bad = (ctypes.c_void_p * 3)(A, A + 2, A)
    assert f(good, 2, bufs_bad, W, 3, 1, A, need, None) == -4
    info = mbq.MbqSequenceInfo()
    assert L.mbq_layer_sequence(good, 2, None, W, 3, 1, A, need, None) == -1
    assert L.mbq_sequence_prepare(good, 2, bufs_bad, W, 3, 1, A, need, None, ctypes.byref(info)) == -4
    assert L.mbq_sequence_prepare(good, 2, bufs, W, 3, 1, A, need, None, None) == -1
    assert L.mbq_sequence_prepare(good, 2, bufs, W, 3, 1, A + 64, need, None, ctypes.byref(info)) == -4
    # mixed bit widths are accepted by the unfused walk only: the workspace
    # query sizes that, and the fused walk's set-up refuses the list
    mixed = _program([(4, 1, 512, 256, A, 0, 1), (6, 0, 256, 512, A, 1, 2)])
    assert L.mbq_sequence_workspace_bytes(mixed, 2, W, 3, 1) > 0
    assert L.mbq_sequence_prepare(mixed, 2, bufs, W, 3, 1, A, need, None, ctypes.byref(info)) == -6
    # run refuses an info block that prepare did not fill
    assert L.mbq_sequence_run(ctypes.byref(info), A, None) == -6
    assert L.mbq_sequence_run(None, A, None) == -1
    assert L.mbq_sequence_check(None, None) == -1


def _op(bits, pro, N, K, i, o, i2=0, w=None):
    return (bits, pro, N, K, A, i, o, i2, 0, w)


def test_sequence_fused_dataflow_rules():
    """Which SwiGLU and weighted-RMSNorm dataflows the fused walk accepts.

    Buffers: 0 x [256]; 1 gate [512]; 2 up [512]; 3 down [256]; 4 o [256];
    5 up' [256].  An accepted list gets past the fused planner and stops at
    the device check (no GPU here); a refused one returns MBQ_ERR_PROGRAM."""
    L = mbq.lib()
    W = (ctypes.c_int64 * 6)(256, 512, 512, 256, 256, 256)
    bufs = (ctypes.c_void_p * 6)(*([A] * 6))
    info = mbq.MbqSequenceInfo()
    Wn, Wn2 = A + 4096, A + 8192      # two sets of norm weights
    WR, SW = mbq.PRO_WRMSNORM_QUANT, mbq.PRO_SWIGLU_QUANT
    gate_up = [_op(4, WR, 512, 256, 0, 1, w=Wn), _op(4, WR, 512, 256, 0, 2, w=Wn)]
    down = _op(4, SW, 256, 512, 1, 3, i2=2)
    cases = {
        "pair in one phase": (gate_up + [down], True),
        "both halves from before the walk": ([down], True),
        "weighted consumers agreeing": (gate_up + [down, _op(4, WR, 256, 256, 3, 4, w=Wn),
                                                  _op(4, WR, 256, 256, 3, 5, w=Wn)], True),
        "weighted consumers disagreeing": (gate_up + [down, _op(4, WR, 256, 256, 3, 4, w=Wn),
                                                     _op(4, WR, 256, 256, 3, 5, w=Wn2)], False),
        "half from before the walk": ([gate_up[0], down], False),
        "halves from two phases": ([gate_up[0], _op(4, WR, 512, 256, 0, 2, w=Wn2), down], False),
        "up read by another op": (gate_up + [down, _op(4, 0, 256, 512, 2, 4)], False),
        "gate read by another op first": (gate_up + [_op(4, 0, 256, 512, 1, 4), down], False),
        "weighted and unweighted consumers": (gate_up + [down, _op(4, WR, 256, 256, 3, 4, w=Wn),
                                                        _op(4, 0, 256, 256, 3, 5)], False),
    }
    for name, (ops, ok) in cases.items():
        prog = _program(ops)
        need = L.mbq_sequence_workspace_bytes(prog, len(ops), W, 6, 2)
        assert need > 0, name          # the unfused walk takes every one of them
        st = L.mbq_sequence_prepare(prog, len(ops), bufs, W, 6, 2, A, need, None, ctypes.byref(info))
        assert (st != -6) == ok, f"{name}: status {st}"
        assert st != 0, name


def test_sequence_fused_buffer_hazards():
    """Op lists whose buffer reuse the fused walk cannot order are refused by it
    (MBQ_ERR_PROGRAM before any device call) and still accepted by the unfused
    walk: an op overwriting a buffer an earlier phase read as an input from
    before the walk, and one buffer written through two different finaliser
    mappings.  Buffers: 0 x [256]; 1 y [512]; 2 w [256]; 3 v [256]."""
    L = mbq.lib()
    W = (ctypes.c_int64 * 4)(256, 512, 256, 256)
    bufs = (ctypes.c_void_p * 4)(*([A] * 4))
    info = mbq.MbqSequenceInfo()
    cases = {
        # x is read from before the walk by the first phase, then overwritten
        "write after an external read": ([_op(4, 1, 512, 256, 0, 1), _op(4, 0, 256, 256, 2, 0)], False),
        # y written first as the first op of its phase, later as the second:
        # its row blocks go to other finalising workgroups the second time
        "rewrite through other finalisers": ([_op(4, 1, 512, 256, 0, 1), _op(4, 1, 256, 256, 0, 2),
                                              _op(4, 0, 256, 256, 2, 3), _op(4, 0, 512, 256, 2, 1)], False),
        # the same rewrite with the same position in its phase is ordered
        "rewrite through the same finalisers": ([_op(4, 1, 512, 256, 0, 1), _op(4, 1, 256, 256, 0, 2),
                                                 _op(4, 0, 512, 256, 2, 1), _op(4, 0, 256, 256, 2, 3)], True),
        # a buffer written in the walk and read back by later phases is fine
        "produced then consumed": ([_op(4, 1, 256, 256, 0, 2), _op(4, 0, 512, 256, 2, 1)], True),
    }
    for name, (ops, ok) in cases.items():
        prog = _program(ops)
        need = L.mbq_sequence_workspace_bytes(prog, len(ops), W, 4, 1)
        assert need > 0, name          # the unfused walk takes every one of them
        st = L.mbq_sequence_prepare(prog, len(ops), bufs, W, 4, 1, A, need, None, ctypes.byref(info))
        assert (st != -6) == ok, f"{name}: status {st}"
        assert st != 0, name


@pytest.mark.parametrize("bits,N,K", [(4, 64, 128), (4, 1, 128), (4, 128, 256), (4, 200, 384), (6, 130, 256),
                                      (4, 1000, 1024), (6, 64 * 7 + 5, 640), (6, 64 * 9, 128), (4, 63, 17408)])
def test_relayout_interleave_schedule(bits, N, K):
    """The padding and row-block interleave steps of the in-place re-layout (block
    rotations by reversal, on the host) turn [codes][scales] into [codes of a row
    block][its scales] per row block, with the padding rows zero."""
    import numpy as np
    rng = np.random.default_rng(N * 7 + K + bits)
    G, Cr = K // 128, K * bits // 8
    R = (N + 63) // 64
    codes = rng.integers(0, 256, (N, Cr), dtype=np.uint8)
    scales = rng.integers(0, 1 << 16, (N, G), dtype=np.uint16)
    total = mbq.lib().mbq_packed_bytes(bits, N, K)
    buf = np.full(total, 0xAB, np.uint8)     # bytes past the canonical data are garbage
    canon = np.concatenate([codes.reshape(-1), scales.reshape(-1).view(np.uint8)])
    buf[:canon.size] = canon
    mbq.relayout_interleave_host(bits, buf, N, K)
    pc = np.zeros((R * 64, Cr), np.uint8)
    pc[:N] = codes
    ps = np.zeros((R * 64, G), np.uint16)
    ps[:N] = scales
    want = np.concatenate([np.concatenate([pc[64 * b:64 * b + 64].reshape(-1),
                                           ps[64 * b:64 * b + 64].reshape(-1).view(np.uint8)])
                           for b in range(R)])
    assert want.size == total
    assert np.array_equal(buf, want)


def test_pack_inplace_validation():
    L = mbq.lib()
    need = L.mbq_packed_bytes(4, 64, 128)
    assert L.mbq_pack_weights_inplace(5, 64, 128, A, need, None) == -3
    assert L.mbq_pack_weights_inplace(4, 64, 128, None, need, None) == -1
    assert L.mbq_pack_weights_inplace(4, 64, 100, A, need, None) == -2
    assert L.mbq_pack_weights_inplace(4, 0, 128, A, need, None) == -2
    assert L.mbq_pack_weights_inplace(4, 64, 128, A + 16, need, None) == -4
    assert L.mbq_pack_weights_inplace(4, 64, 128, A, need - 1, None) == -5
    assert L.mbq_relayout_interleave_host(4, 64, 128, None, need) == -1
