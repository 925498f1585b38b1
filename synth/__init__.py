"""Seeded synthetic inputs for the skinny W4A8/W6A8 linear and its decode-step walk.

This module only draws random numbers and lays them out as bytes; it holds none
of the method's arithmetic (no decoding, quantisation, dot products or
rescaling).  Both the CPU oracle and the HIP path are fed from here, so they
see identical bytes.

Distributions follow the workloads described for the "Doubling LLM token rates
in ComfyUI" page (section "What is the bottleneck?": a dense, often square
weight matrix times one activation row, or a thin block of 3 rows for a
multi-token-prediction verify step):

* activations: fp32 N(0, 1), rounded to bf16 (round to nearest even);
* weight codes: uniform over the whole code range.  Two independent uniform
  int4 codes per byte form a uniform byte, and four uniform int6 codes per
  three bytes form a uniform 24-bit word, so canonical weight bytes are simply
  uniform random bytes;
* group scales: fp32 U(0.005, 0.02) rounded to fp16, one per 128 weights
  along K.

* RMSNorm weights (the "real" dataflow's weighted norms): fp32 U(0.5, 1.5)
  rounded to bf16, one per input column.

Seeds: matrix i of a weight set uses seed ``1 + i`` (codes drawn first, then
scales); an activation block of M rows uses seed ``1_000_000 + M``; the norm
weights in front of the attention (mlp) projections of layer l use seed
``2_000_000 + 2 * l`` (``+ 1``).
"""
from __future__ import annotations

import numpy as np

GROUP = 128
ACT_SEED_BASE = 1_000_000


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def activations(M: int, K: int, seed: int | None = None) -> np.ndarray:
    """bf16 bit patterns, shape [M][K], from fp32 N(0,1)."""
    rng = _rng(ACT_SEED_BASE + M if seed is None else seed)
    return f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


def norm_weights(K: int, seed: int) -> np.ndarray:
    """bf16 bit patterns [K] of RMSNorm weights, from fp32 U(0.5, 1.5)."""
    return f32_to_bf16_bits(_rng(seed).uniform(0.5, 1.5, K).astype(np.float32))


def canon_row_bytes(bits: int, K: int) -> int:
    """Bytes per weight row in the canonical (checkpoint-like) layout."""
    if bits not in (4, 6):
        raise ValueError("bits must be 4 or 6")
    return K * bits // 8


def weights(bits: int, N: int, K: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Canonical weight bytes u8[N][K*bits/8] and fp16 group scales [N][K/128]."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    rng = _rng(seed)
    nb = canon_row_bytes(bits, K)
    codes = np.frombuffer(rng.bytes(N * nb), dtype=np.uint8).reshape(N, nb)
    scales = rng.uniform(0.005, 0.02, size=(N, K // GROUP)).astype(np.float32).astype(np.float16)
    return codes, scales


def scales_only(N: int, K: int, seed: int) -> np.ndarray:
    return _rng(seed).uniform(0.005, 0.02, size=(N, K // GROUP)).astype(np.float32).astype(np.float16)


# ---------------------------------------------------------------------------
# Decode-step weight sets.  Each layer lists (name, K, N) in execution order;
# the walk is described by synth.layer_program().

def layer_shapes_9b() -> list[tuple[str, int, int]]:
    """9B-shaped decoder layer: hidden 4096, intermediate 12288."""
    H, I, KV = 4096, 12288, 1024
    return [("q", H, H), ("k", H, KV), ("v", H, KV), ("o", H, H),
            ("gate", H, I), ("up", H, I), ("down", I, H)]


def layer_shapes_27b() -> list[tuple[str, int, int]]:
    """27B-shaped decoder layer: hidden 5120, intermediate 17408.

    The pages give no head counts.  The query projection carries the query and
    a per-head output gate (2 x 64 heads x 128), the output projection reads
    the 8192-wide attention output, and k/v are 8 heads x 128.  This is the
    shape choice whose packed int4 weights land nearest the ~14 GB per token
    stated on the page (section "What is the bottleneck?").
    """
    H, I = 5120, 17408
    return [("q", H, 16384), ("k", H, 1024), ("v", H, 1024), ("o", 8192, H),
            ("gate", H, I), ("up", H, I), ("down", I, H)]


WEIGHT_SETS = {
    "9b": (layer_shapes_9b, 36),
    "27b": (layer_shapes_27b, 64),
}


def weight_set(name: str, n_layers: int | None = None) -> list[tuple[str, int, int, int]]:
    """Flat list of (name, K, N, seed) for every matrix of a decode step."""
    shapes_fn, default_layers = WEIGHT_SETS[name]
    L = default_layers if n_layers is None else n_layers
    out = []
    i = 0
    for layer in range(L):
        for nm, K, N in shapes_fn():
            out.append((f"L{layer}.{nm}", K, N, 1 + i))
            i += 1
    return out


def weight_bytes(bits: int, shapes) -> int:
    """Algorithmic weight-read bytes: packed codes plus fp16 group scales."""
    tot = 0
    for s in shapes:
        K, N = s[1], s[2]
        tot += N * K * bits // 8 + N * (K // GROUP) * 2
    return tot


# Buffer and op indices of the decode-step walk.  Per layer:
#   x --RMSNorm+quant--> q, k, v      (k, v written, unread: KV-append stand-ins)
#   q[:, :K_o] --quant--> o
#   o --quant--> gate, up              (up written, unread: SwiGLU partner stand-in)
#   gate --quant--> down --> x of the next layer
#
# The "real" dataflow (dataflow="swiglu") puts the norms and gate of a decoder
# layer in front of the quantisations instead:
#   x --weighted RMSNorm+quant--> q, k, v
#   q[:, :K_o] --quant--> o
#   o --weighted RMSNorm+quant--> gate, up
#   (gate, up) --SwiGLU+quant--> down --> x of the next layer
BUF_NAMES = ["x", "q", "k", "v", "o", "gate", "up", "down"]
PRO_QUANT = 0
PRO_RMSNORM_QUANT = 1
PRO_WRMSNORM_QUANT = 2
PRO_SWIGLU_QUANT = 3
NORM_SEED_BASE = 2_000_000


def layer_program(shapes_fn, n_layers: int, distinct_buffers: bool = False, dataflow: str = "plain"):
    """Op list of a decode-step walk.

    Returns (ops, buf_widths) where ops are dicts with keys
    name, K, N, in_buf, out_buf, prologue, matrix (index into the weight set),
    and for dataflow="swiglu" also in_buf2 (the down op's up buffer) and
    norm_seed (the seed of the op's RMSNorm weights, see norm_weights).
    With distinct_buffers every op writes a buffer of its own so that every
    intermediate survives the walk (used by parity tests).  Otherwise the eight
    buffers of BUF_NAMES are reused by every layer: layer 0 reads buffer "x",
    and every later layer reads the "down" buffer written by the layer before.
    """
    if dataflow not in ("plain", "swiglu"):
        raise ValueError("dataflow must be 'plain' or 'swiglu'")
    sw = dataflow == "swiglu"
    # (name, input, prologue); the input None is the layer's x
    plan = (("q", None, PRO_WRMSNORM_QUANT if sw else PRO_RMSNORM_QUANT),
            ("k", None, PRO_WRMSNORM_QUANT if sw else PRO_RMSNORM_QUANT),
            ("v", None, PRO_WRMSNORM_QUANT if sw else PRO_RMSNORM_QUANT),
            ("o", "q", PRO_QUANT),
            ("gate", "o", PRO_WRMSNORM_QUANT if sw else PRO_QUANT),
            ("up", "o", PRO_WRMSNORM_QUANT if sw else PRO_QUANT),
            ("down", "gate", PRO_SWIGLU_QUANT if sw else PRO_QUANT))

    def extra(layer, nm, buf_of):
        if not sw:
            return {}
        if nm == "down":
            return {"in_buf2": buf_of("up")}
        if nm in ("q", "k", "v"):
            return {"norm_seed": NORM_SEED_BASE + 2 * layer}
        if nm in ("gate", "up"):
            return {"norm_seed": NORM_SEED_BASE + 2 * layer + 1}
        return {}

    shapes = shapes_fn()
    widths = {}
    ops = []
    mi = 0
    H = shapes[0][1]
    if distinct_buffers:
        bufw = [H]
        cur_x = 0
        for layer in range(n_layers):
            idx = {}
            for nm, K, N in shapes:
                bufw.append(N)
                idx[nm] = len(bufw) - 1
            for nm, in_name, pro in plan:
                K, N = next((k, n) for (n_, k, n) in shapes if n_ == nm)
                src = cur_x if in_name is None else idx[in_name]
                ops.append(dict(name=f"L{layer}.{nm}", K=K, N=N, in_buf=src, out_buf=idx[nm],
                                prologue=pro, matrix=mi, **extra(layer, nm, lambda b: idx[b])))
                mi += 1
            cur_x = idx["down"]
        return ops, bufw
    sh = {nm: (K, N) for nm, K, N in shapes}
    bufw = [H, sh["q"][1], sh["k"][1], sh["v"][1], sh["o"][1], sh["gate"][1], sh["up"][1], sh["down"][1]]
    B = {n: i for i, n in enumerate(BUF_NAMES)}
    for layer in range(n_layers):
        src = B["x"] if layer == 0 else B["down"]
        for nm, in_name, pro in plan:
            K, N = sh[nm]
            ib = src if in_name is None else B[in_name]
            ops.append(dict(name=f"L{layer}.{nm}", K=K, N=N, in_buf=ib, out_buf=B[nm],
                            prologue=pro, matrix=mi, **extra(layer, nm, lambda b: B[b])))
            mi += 1
    return ops, bufw
