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


@pytest.fixture(params=["kernel", "inline"])
def combine(request, monkeypatch):
    """Both combines of the splits: the second kernel (the default) and the one
    at the end of a cooperative split launch (MBQ_ATTN_COMBINE=inline)."""
    if request.param == "inline":
        monkeypatch.setenv("MBQ_ATTN_COMBINE", "inline")
    else:
        monkeypatch.delenv("MBQ_ATTN_COMBINE", raising=False)
    return request.param


def _run(q, k, v, P, ws=None):
    import torch
    out = mbq.decode_attention(dev(q).view(torch.bfloat16), dev(k).view(torch.bfloat16),
                               dev(v).view(torch.bfloat16), P, ws=ws)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("P", [0, 1, 63, 64, 65, 200, 1000])
@pytest.mark.parametrize("M,n_q,n_kv,D", [(1, 1, 1, 64), (1, 8, 1, 128), (2, 4, 2, 256), (3, 6, 3, 64),
                                          (8, 8, 1, 256), (5, 16, 4, 128), (8, 16, 2, 64), (5, 8, 1, 256)])
def test_decode_attention_matches_oracle(M, n_q, n_kv, D, P, combine):
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


def test_decode_attention_workspace_reused(combine):
    """Calls of different P (so different split counts, 1 at P = 10) on one
    workspace -- garbage for the second-kernel combine, zero-filled for the
    in-launch one, whose counters must be back at zero after every call --
    and a repeated call gives the same bits."""
    import torch
    M, n_q, n_kv, D = 4, 8, 2, 128
    need = max(mbq.attention_workspace_bytes(M, n_q, n_kv, D, P) for P in (3000, 10, 40000))
    ws = torch.full((need,), 0 if combine == "inline" else 0xA5, dtype=torch.uint8, device="cuda")
    first = {}
    for P in (3000, 10, 40000, 3000, 40000):
        L = P + M
        q, k, v = _inputs(M, n_q, n_kv, D, L, seed=P)
        got = _run(q, k, v, P, ws=ws)
        assert_close_bf16(got, oracle.decode_attention(q, k, v, P), f"P={P}")
        if P in first:
            assert np.array_equal(got, first[P]), f"P={P} repeated"
        first[P] = got


@pytest.mark.parametrize("M", [1, 4, 8])
def test_decode_attention_27b_shape(M, combine):
    """The 27B-shaped attention layer: 32 query heads, 4 key/value heads of 256,
    a 32768-token prefix (M = 4: two row tiles, two workgroups per CU)."""
    n_q, n_kv, D, P = 32, 4, 256, 32768
    L = P + M
    q, k, v = _inputs(M, n_q, n_kv, D, L, seed=77 + M)
    assert_close_bf16(_run(q, k, v, P), oracle.decode_attention(q, k, v, P), f"27B M={M}")


@pytest.mark.parametrize("P", [32767, 40895, 40960])
def test_decode_attention_split_remainders(P, combine):
    """Cache lengths whose blocks do not divide evenly over the splits: the
    last (blocks mod splits) splits take one more block.  On the 27B layer
    shape with 128 splits, 32767 + 1 positions are 512 blocks (none left
    over), 40895 + 1 are 639 (all splits but one take one more) and 40960 + 1
    are 641 (only the last takes one more: the one-row tail)."""
    n_q, n_kv, D, M = 32, 4, 256, 1
    q, k, v = _inputs(M, n_q, n_kv, D, P + M, seed=P)
    assert_close_bf16(_run(q, k, v, P), oracle.decode_attention(q, k, v, P), f"27B P={P}")


@pytest.mark.parametrize("M,n_q,n_kv,D", [(1, 16, 4, 128), (8, 16, 4, 128), (1, 8, 2, 64), (8, 8, 2, 64),
                                          (5, 8, 8, 256)])
def test_decode_attention_long_prefix_other_shapes(M, n_q, n_kv, D, combine):
    """A long prefix that is not a whole number of blocks, over other head
    sizes, group sizes and row counts: every form (one, two or four row tiles;
    64- or 32-position blocks) deals its blocks over many splits with some
    left over."""
    P = 20011
    q, k, v = _inputs(M, n_q, n_kv, D, P + M, seed=M * 1000 + D)
    assert_close_bf16(_run(q, k, v, P), oracle.decode_attention(q, k, v, P), f"M={M} D={D} n_kv={n_kv}")


@pytest.mark.parametrize("P", [1100, 2048, 4000])
@pytest.mark.parametrize("M,n_q,n_kv,D", [(1, 32, 4, 256), (8, 32, 4, 256), (3, 8, 2, 128), (5, 8, 1, 64)])
def test_decode_attention_merge_group_widths(M, n_q, n_kv, D, P, combine):
    """Split counts for every width of the merge's lane groups.  A group of
    tpq lanes sums a run of four outputs, at most 8 splits per lane, and a
    wave's groups are interleaved over its lanes, so each tpq is its own lane
    mapping.  These cache lengths give 9 splits (tpq 2), 17 (tpq 4, most
    splits one block longer) and 32 (tpq 4, the most it covers); the other
    tests cover up to 8 splits (tpq 1), 40 to 64 (tpq 8) and 128 (tpq 16)."""
    q, k, v = _inputs(M, n_q, n_kv, D, P + M, seed=P + 10 * M + D)
    assert_close_bf16(_run(q, k, v, P), oracle.decode_attention(q, k, v, P), f"M={M} D={D} P={P}")


def test_decode_attention_graph_replays(combine):
    """The attention captured in a HIP graph (two launches, or one cooperative
    launch with the merge inside): replays on queries written between them
    equal eager calls bit for bit."""
    import torch
    M, n_q, n_kv, D, P = 2, 8, 2, 128, 5000
    L = P + M
    _, k, v = _inputs(M, n_q, n_kv, D, L, seed=9)
    kd, vd = dev(k).view(torch.bfloat16), dev(v).view(torch.bfloat16)
    qs = [dev(_inputs(M, n_q, n_kv, D, 16, seed=40 + i)[0]).view(torch.bfloat16) for i in range(3)]
    qbuf = torch.empty_like(qs[0])
    out = torch.empty((M, n_q, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(mbq.attention_workspace_bytes(M, n_q, n_kv, D, P), dtype=torch.uint8, device="cuda")
    eager = []
    for qi in qs:
        qbuf.copy_(qi)
        mbq.decode_attention(qbuf, kd, vd, P, out=out, ws=ws)
        torch.cuda.synchronize()
        eager.append(host(out))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mbq.decode_attention(qbuf, kd, vd, P, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mbq.decode_attention(qbuf, kd, vd, P, out=out, ws=ws)
    for i in (1, 0, 2, 1):
        qbuf.copy_(qs[i])
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), eager[i]), f"replay of query {i}"
