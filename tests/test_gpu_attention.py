"""GPU parity of the split-prefix decode attention against the oracle
("Paying attention to the attention!" on the page "Doubling LLM token rates in
ComfyUI"), through the C ABI."""
import numpy as np
import pytest

import memory_bound_quantised_amd as mbq
import oracle
import synth
from tests.gpu_util import assert_close_bf16, dev, host

pytestmark = pytest.mark.gpu


def _inputs(M, n_q, n_kv, D, L, seed):
    rng = np.random.default_rng(seed)
    q = synth.f32_to_bf16_bits(rng.standard_normal((M, n_q, D), dtype=np.float32))
    k = synth.f32_to_bf16_bits(rng.standard_normal((n_kv, L, D), dtype=np.float32))
    v = synth.f32_to_bf16_bits(rng.standard_normal((n_kv, L, D), dtype=np.float32))
    return q, k, v


def _run(q, k, v, P, ws=None):
    import torch
    out = mbq.decode_attention(dev(q).view(torch.bfloat16), dev(k).view(torch.bfloat16),
                               dev(v).view(torch.bfloat16), P, ws=ws)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("P", [0, 1, 63, 64, 65, 200, 1000])
@pytest.mark.parametrize("M,n_q,n_kv,D", [(1, 1, 1, 64), (1, 8, 1, 128), (2, 4, 2, 256), (3, 6, 3, 64),
                                          (8, 8, 1, 256), (5, 16, 4, 128), (8, 16, 2, 64), (5, 8, 1, 256)])
def test_decode_attention_matches_oracle(M, n_q, n_kv, D, P):
    L = P + M + 5
    q, k, v = _inputs(M, n_q, n_kv, D, L, seed=P * 31 + M * 7 + D)
    got = _run(q, k, v, P)
    assert_close_bf16(got, oracle.decode_attention(q, k, v, P), f"M={M} P={P}")


def test_decode_attention_causal_rows_and_heads_exactly():
    """Uniform scores and one-hot values: every output is 1/(positions attended)
    on exactly the attended positions, so a wrong mask or head mapping shows."""
    import torch
    M, n_q, n_kv, D, P = 8, 16, 2, 64, 40
    L = P + M
    q = np.zeros((M, n_q, D), np.uint16)
    k = synth.f32_to_bf16_bits(np.random.default_rng(2).standard_normal((n_kv, L, D), dtype=np.float32))
    vf = np.zeros((n_kv, L, D), np.float32)
    for g in range(n_kv):
        for p in range(L):
            vf[g, p, p] = g + 1
    v = synth.f32_to_bf16_bits(vf)
    got = _run(q, k, v, P)
    assert np.array_equal(got, oracle.decode_attention(q, k, v, P))


def test_decode_attention_workspace_reused():
    """Calls of different P on one workspace, which starts out as garbage."""
    import torch
    M, n_q, n_kv, D = 4, 8, 2, 128
    need = max(mbq.attention_workspace_bytes(M, n_q, n_kv, D, P) for P in (3000, 10))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for P in (3000, 10, 3000):
        L = P + M
        q, k, v = _inputs(M, n_q, n_kv, D, L, seed=P)
        assert_close_bf16(_run(q, k, v, P, ws=ws), oracle.decode_attention(q, k, v, P), f"P={P}")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_decode_attention_27b_shape(M):
    """The 27B-shaped attention layer: 32 query heads, 4 key/value heads of 256,
    a 32768-token prefix (M = 4: two row tiles, two workgroups per CU)."""
    n_q, n_kv, D, P = 32, 4, 256, 32768
    L = P + M
    q, k, v = _inputs(M, n_q, n_kv, D, L, seed=77 + M)
    assert_close_bf16(_run(q, k, v, P), oracle.decode_attention(q, k, v, P), f"27B M={M}")
