"""Helpers for the GPU parity tests: host <-> device copies and the tolerance."""
import numpy as np

import memory_bound_quantised_amd as mbq
import oracle
import synth

# bf16 outputs: |y_gpu - y_oracle| <= ATOL + RTOL * |y_oracle|
ATOL = 1e-3
RTOL = 1e-2


def dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:                       # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def host(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_f64(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def assert_close_bf16(y_gpu_bits, y_ref_bits, what=""):
    g = bf16_f64(y_gpu_bits)
    r = bf16_f64(y_ref_bits)
    err = np.abs(g - r)
    bound = ATOL + RTOL * np.abs(r)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} outputs out of tolerance, first at {bad[0].tolist()}: "
                           f"gpu {g[tuple(bad[0])]} oracle {r[tuple(bad[0])]}")
    assert np.all(np.isfinite(g))


def packed_on_device(bits, canon, scales, N, K):
    return mbq.pack_weights(bits, dev(canon), dev(scales), N, K)


def oracle_rows(bits, x_bf16, prologue, canon, scales, rows):
    """Oracle outputs of an op restricted to output rows `rows` (rows are independent)."""
    return oracle.op(bits, x_bf16, prologue, canon[rows], scales[rows])


def sample_rows(rng, N, k=256):
    if N <= k:
        return np.arange(N)
    r = rng.choice(np.arange(1, N - 1), size=k - 2, replace=False)
    return np.sort(np.concatenate([[0, N - 1], r]))
