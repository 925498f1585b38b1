"""The allocation-free linear (mbq_linear_noalloc) against the workspace linear.

mbq_linear_noalloc runs the same kernels as mbq_w4a8_linear / mbq_w6a8_linear
with its split-K scratch in the library's own device array; its outputs must
equal the workspace entry point's bitwise, call after call (the array keeps
the previous call's contents), and agree with the oracle within the linear's
tolerance.  This file is collected last so that a failure here cannot hide
the other GPU tests."""
import numpy as np
import pytest

import memory_bound_quantised_amd as mbq
import oracle
import synth
from tests.gpu_util import assert_close_bf16, dev, host, packed_on_device, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mbq.lib()
    yield
    torch.cuda.synchronize()


def _case(bits, M, N, K, seed):
    import torch
    canon, S = synth.weights(bits, N, K, seed=seed)
    x = synth.activations(M, K, seed=seed + 1)
    q, s = oracle.quantize_act(x)
    packed = packed_on_device(bits, canon, S, N, K)
    qd, sd = dev(q), dev(s)
    y_ref = host(mbq.linear(bits, qd, sd, packed, N))            # the workspace entry point
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = host(mbq.linear_noalloc(bits, qd, sd, packed, N, out))
    torch.cuda.synchronize()
    assert np.array_equal(y, y_ref), f"W{bits} M={M} {N}x{K}: differs from mbq_w{bits}a8_linear"
    rows = sample_rows(np.random.default_rng(seed), N)
    assert_close_bf16(y[:, rows], oracle.linear(bits, q, s, canon[rows], S[rows]), f"W{bits} M={M} {N}x{K}")


def test_noalloc_matches_workspace_linear_two_calls():
    """A large split-K call, then a smaller one on the same device array."""
    _case(4, 3, 5120, 17408, seed=41)     # 16 splits per row block, 80 row blocks
    _case(6, 1, 1000, 4096, seed=42)      # fewer row blocks and splits


def test_noalloc_repeated_and_shapes():
    """More calls in a row over shapes whose counters and partials overlap."""
    for i, (bits, M, N, K) in enumerate([(4, 8, 17408, 5120), (4, 1, 4096, 4096), (6, 4, 200, 1152),
                                         (4, 2, 64, 128), (6, 3, 4096, 12288)]):
        _case(bits, M, N, K, seed=100 + i)
