"""Pins of the decode-attention oracle ("Paying attention to the attention!"
on the page "Doubling LLM token rates in ComfyUI"): closed forms and
invariants, none of them a retyping of the oracle's formula."""
import math

import numpy as np
import pytest

import oracle
import synth


def bf16(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def val(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("M,n_q,n_kv,P", [(1, 1, 1, 0), (1, 4, 2, 7), (3, 8, 2, 5), (8, 8, 1, 30), (5, 6, 3, 0)])
def test_uniform_scores_average_exactly_the_attended_positions(M, n_q, n_kv, P):
    """q = 0 makes every score 0, and v_p = (g+1) e_p (a one-hot per position,
    scaled by the key/value head) turns the output into the attended set:
    token i of a head in group g gives (g+1)/(P+i+1) at d <= P+i and 0 beyond."""
    D = 64
    L = P + M + 3
    assert L <= D
    q = np.zeros((M, n_q, D), np.uint16)
    k = bf16(np.random.default_rng(1).standard_normal((n_kv, L, D)))
    v = np.zeros((n_kv, L, D), np.float32)
    for g in range(n_kv):
        for p in range(L):
            v[g, p, p] = g + 1
    o = oracle.decode_attention(q, k, bf16(v), P)
    qpg = n_q // n_kv
    for i in range(M):
        n = P + i + 1
        for h in range(n_q):
            g = h // qpg
            want = np.zeros(D, np.uint16)
            want[:n] = oracle.f64_to_bf16((g + 1) / n)
            assert np.array_equal(o[i, h], want), (i, h)


@pytest.mark.parametrize("c,D", [(4.0, 64), (-3.0, 16), (10.0, 256)])
def test_two_keys_weight_is_the_logistic_of_the_scaled_score(c, D):
    """Keys 0 and c e_0 against q = e_0: the second position's weight is
    1 / (1 + exp(-c / sqrt(D))); with v = 0 and 1 that weight is the output."""
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 2, D), np.float32)
    k[0, 1, 0] = c
    v = np.zeros((1, 2, D), np.float32)
    v[0, 1, :] = 1.0
    o = oracle.decode_attention(bf16(q), bf16(k), bf16(v), 1)
    w = 1.0 / (1.0 + math.exp(-c / math.sqrt(D)))
    assert np.all(o == oracle.f64_to_bf16(w))


def test_prefix_order_does_not_matter_and_later_positions_are_unseen():
    """Swapping two prefix positions (key and value together) leaves every
    output unchanged; changing the last new token's key and value changes
    only the last row."""
    rng = np.random.default_rng(3)
    M, n_q, n_kv, D, P = 4, 4, 2, 32, 9
    L = P + M
    q = bf16(rng.standard_normal((M, n_q, D)))
    k = bf16(rng.standard_normal((n_kv, L, D)))
    v = bf16(rng.standard_normal((n_kv, L, D)))
    o = oracle.decode_attention(q, k, v, P)
    k2, v2 = k.copy(), v.copy()
    k2[:, [2, 7]] = k[:, [7, 2]]
    v2[:, [2, 7]] = v[:, [7, 2]]
    assert np.array_equal(oracle.decode_attention(q, k2, v2, P), o)
    k3, v3 = k.copy(), v.copy()
    k3[:, L - 1] = bf16(rng.standard_normal((n_kv, D)))
    v3[:, L - 1] = bf16(rng.standard_normal((n_kv, D)))
    o3 = oracle.decode_attention(q, k3, v3, P)
    assert np.array_equal(o3[:M - 1], o[:M - 1])
    assert not np.array_equal(o3[M - 1], o[M - 1])


def test_brute_force_small_case():
    """A 2-token, 2-head case summed term by term in Python floats."""
    rng = np.random.default_rng(5)
    M, n_q, n_kv, D, P = 2, 2, 1, 8, 3
    L = P + M
    q = bf16(rng.standard_normal((M, n_q, D)))
    k = bf16(rng.standard_normal((n_kv, L, D)))
    v = bf16(rng.standard_normal((n_kv, L, D)))
    o = oracle.decode_attention(q, k, v, P)
    qv, kv, vv = val(q), val(k), val(v)
    for i in range(M):
        for h in range(n_q):
            s = [sum(qv[i, h, d] * kv[0, p, d] for d in range(D)) / math.sqrt(D) for p in range(P + i + 1)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            for d in range(D):
                want = sum(w[p] * vv[0, p, d] for p in range(len(w))) / sum(w)
                assert o[i, h, d] == oracle.f64_to_bf16(want)
