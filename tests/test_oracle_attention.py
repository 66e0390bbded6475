"""Pins of the oracle's joint-softmax attention (no GPU).

What fixes the expected values:
  * when the budget covers every candidate, window + top-k is the whole causal
    domain, so the result must equal dense causal attention, here computed by
    torch's scaled_dot_product_attention in float64 (a library routine);
  * special cases: one visible entry gives its value row; equal logits give the
    mean of the value rows; an empty set gives 0 and lse = -inf;
  * the dropped-mass bound: if the kept set S misses dense attention mass eps
    and every value row has norm <= V, then ||o_dense - o_S|| <= 2 eps V
    (HySparse2 page, section 18 and the supplementary "why it can work"
    derivation: renormalised output over the kept positions);
  * FP4 storage: attention over E2M1 codes equals attention over the same
    values dequantised independently with torch's E4M3 decoder.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F


def _sdpa_dense(q, K, V, t_list, hkv, scale):
    """q [S, R, Hq, d] for rows at positions t_list of one sequence; K, V
    [L, Hkv, d]. Dense causal attention through torch SDPA (float64)."""
    S, R, Hq, d = q.shape
    G = Hq // hkv
    out = torch.zeros(S, R, Hq, V.shape[-1], dtype=torch.float64)
    lse = torch.zeros(S, R, Hq, dtype=torch.float64)
    for r, t in enumerate(t_list):
        k = K[: t + 1].double()  # [n, Hkv, d]
        v = V[: t + 1].double()
        for h in range(Hq):
            g = h // G
            qq = q[:, r, h].double()[:, None, :]  # [S, 1, d]
            o = F.scaled_dot_product_attention(qq[None], k[:, g][None, None].expand(1, S, -1, -1),
                                               v[:, g][None, None].expand(1, S, -1, -1),
                                               scale=scale)
            out[:, r, h] = o[0, :, 0]
            lse[:, r, h] = torch.logsumexp(scale * (qq[:, 0] @ k[:, g].T), dim=-1)
    return out.numpy(), lse.numpy()


@pytest.mark.parametrize("window", [0, 5, 64])
def test_full_budget_equals_dense(orc, window):
    g = torch.Generator().manual_seed(20 + window)
    L, Hq, Hkv, d, S = 48, 4, 2, 16, 2
    q = torch.randn(S, L, Hq, d, generator=g)
    K = torch.randn(1, L, Hkv, d, generator=g)
    V = torch.randn(1, L, Hkv, 24, generator=g)
    t_list = list(range(L))
    so, po, sl = np.zeros(L, np.int32), np.arange(L, dtype=np.int32), np.array([L], np.int32)
    scale = 1.0 / math.sqrt(d)
    # select everything outside the window
    idx = np.full((L, L), -1, np.int32)
    cnt = np.zeros(L, np.int32)
    for t in t_list:
        c = list(range(max(0, t + 1 - window)))
        idx[t, :len(c)] = c
        cnt[t] = len(c)
    o, lse = orc.attention(so, po, sl, 1, window, q, K, V, idx, cnt, scale=float(np.float32(scale)))
    ref, rlse = _sdpa_dense(q, K[0], V[0], t_list, Hkv, float(np.float32(scale)))
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, rlse, rtol=1e-12, atol=1e-12)


def test_special_cases(orc):
    g = torch.Generator().manual_seed(30)
    L, Hq, d = 10, 2, 8
    K = torch.randn(1, L, 1, d, generator=g)
    V = torch.randn(1, L, 1, d, generator=g)
    so, sl = np.zeros(3, np.int32), np.array([L], np.int32)
    # row 0 at t=0 sees one entry -> its value row
    # row 1 has q = 0 -> equal logits -> mean of the visible value rows
    # row 2 is a padding row -> empty
    so[2] = -1
    po = np.array([0, 6, 3], np.int32)
    q = torch.randn(1, 3, Hq, d, generator=g)
    q[0, 1] = 0
    o, lse = orc.attention(so, po, sl, 1, 100, q, K, V, None, None, scale=0.5)
    assert np.allclose(o[0, 0], V[0, 0, 0].double().numpy()[None].repeat(Hq, 0), atol=0, rtol=0)
    mean = V[0, :7, 0].double().mean(0).numpy()
    assert np.allclose(o[0, 1], mean[None].repeat(Hq, 0), rtol=1e-14, atol=1e-14)
    assert np.allclose(lse[0, 1], math.log(7.0), rtol=1e-14)
    assert np.all(o[0, 2] == 0) and np.all(np.isneginf(lse[0, 2]))


def test_gqa_head_map(orc):
    """Query head h reads KV head floor(h * Hkv / Hq): give every KV head a
    constant distinct value row and check which one each query head returns."""
    L, Hq, Hkv, d = 5, 8, 4, 4
    K = torch.zeros(1, L, Hkv, d)
    V = torch.arange(Hkv, dtype=torch.float32)[None, None, :, None].expand(1, L, Hkv, d).clone()
    q = torch.randn(1, 1, Hq, d)
    o, _ = orc.attention(np.zeros(1, np.int32), np.array([L - 1], np.int32),
                         np.array([L], np.int32), 1, L, q, K, V, None, None, scale=1.0)
    for h in range(Hq):
        assert np.allclose(o[0, 0, h], h * Hkv // Hq, rtol=1e-14, atol=0)


@pytest.mark.parametrize("concentrated", [False, True])
def test_dropped_mass_bound(orc, concentrated):
    rng = np.random.default_rng(40 + concentrated)
    L, d = 300, 32
    if concentrated:  # low-rank queries/keys make attention peaked
        u = rng.standard_normal((L, 2))
        K = torch.tensor(u @ rng.standard_normal((2, d)) * 3.0)
        q = torch.tensor(u[-1:] @ rng.standard_normal((2, d)) * 3.0)
    else:
        K = torch.tensor(rng.standard_normal((L, d)))
        q = torch.tensor(rng.standard_normal((1, d)))
    V = torch.tensor(rng.standard_normal((L, d)))
    Kt, Vt, qt = K.float()[None, :, None], V.float()[None, :, None], q.float()[None, :, None]
    so, po, sl = np.zeros(1, np.int32), np.array([L - 1], np.int32), np.array([L], np.int32)
    scale = 1.0 / math.sqrt(d)
    dense, _ = orc.attention(so, po, sl, 1, L, qt, Kt, Vt, None, None, scale=scale)
    logits = (qt[0, 0, 0].double() @ Kt[0, :, 0].double().T) * float(np.float32(scale))
    p = torch.softmax(logits, 0).numpy()
    vmax = np.linalg.norm(Vt[0, :, 0].double().numpy(), axis=1).max()
    for trial in range(20):
        m = int(rng.integers(1, L))
        keep = np.sort(rng.choice(L, m, replace=False)).astype(np.int32)
        if trial % 2:  # keep the heaviest positions
            keep = np.sort(np.argsort(-p)[:m]).astype(np.int32)
        o, _ = orc.attention(so, po, sl, 1, 0, qt, Kt, Vt, keep[None], np.array([m], np.int32),
                             scale=scale)
        eps = 1.0 - p[keep].sum()
        err = np.linalg.norm(o[0, 0, 0] - dense[0, 0, 0])
        assert err <= 2 * eps * vmax + 1e-12


def test_fp4_equals_dequantised(orc):
    import synth

    g_seed = 50
    L, Hkv, d, Hq = 40, 1, 64, 4
    x = synth.normal((1, L, Hkv, d), seed=g_seed)
    codes, scales = synth.fp4_encode(x)
    # independent dequantisation: E2M1 by table, E4M3 by torch
    grid = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=torch.float64)
    lo, hi = codes & 15, codes >> 4
    nib = torch.stack([lo, hi], dim=-1).reshape(1, L, Hkv, d).long()
    val = grid[nib & 7] * torch.where((nib & 8) > 0, -1.0, 1.0).double()
    sc = scales.view(torch.float8_e4m3fn).double().repeat_interleave(16, dim=-1)
    deq = (val * sc).to(torch.bfloat16)
    q = synth.normal((1, 3, Hq, d), seed=51, dtype=torch.bfloat16)
    so, po, sl = np.zeros(3, np.int32), np.array([0, 20, 39], np.int32), np.array([L], np.int32)
    idx = np.array([[-1] * 8, [1, 3, 5, 7, 9, -1, -1, -1], [0, 2, 4, 8, 16, 30, 31, 32]], np.int32)
    cnt = np.array([0, 5, 8], np.int32)
    o4, l4 = orc.attention(so, po, sl, 1, 4, q, codes, None, idx, cnt, k_scale=scales,
                           v_from_k=True, dv=d, fp4=True, hkv=Hkv)
    ob, lb = orc.attention(so, po, sl, 1, 4, q, deq, None, idx, cnt, v_from_k=True, dv=d)
    assert np.array_equal(o4, ob) and np.array_equal(l4, lb)


def test_window_union_counts_once(orc):
    """A selected position inside the window is not counted twice."""
    L, d = 12, 4
    g = torch.Generator().manual_seed(60)
    K = torch.randn(1, L, 1, d, generator=g)
    V = torch.randn(1, L, 1, d, generator=g)
    q = torch.randn(1, 1, 2, d, generator=g)
    so, po, sl = np.zeros(1, np.int32), np.array([L - 1], np.int32), np.array([L], np.int32)
    a, _ = orc.attention(so, po, sl, 1, 3, q, K, V, np.array([[2, 5]], np.int32),
                         np.array([2], np.int32), scale=0.3)
    b, _ = orc.attention(so, po, sl, 1, 3, q, K, V, np.array([[2, 5, 10, 11]], np.int32),
                         np.array([4], np.int32), scale=0.3)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("window", [0, 7])
def test_latent_v_from_k_equals_dense(orc, window):
    """Latent rows (MLA, "Lecture 10", section 5.1): K is the whole row of
    d_qk channels and V its first d_v < d_qk channels.  With the budget
    covering every candidate, the oracle's v_from_k branch must equal dense
    causal attention whose V is the slice K[..., :d_v], here through torch's
    SDPA in float64.  d_qk = 40 and d_v = 24 keep a row-stride mix-up between
    the two widths visible (every row after the first would be misread)."""
    g = torch.Generator().manual_seed(70 + window)
    L, Hq, dqk, dv, S = 30, 4, 40, 24, 2
    q = torch.randn(S, L, Hq, dqk, generator=g).to(torch.bfloat16)
    K = torch.randn(1, L, 1, dqk, generator=g).to(torch.bfloat16)
    so, po, sl = np.zeros(L, np.int32), np.arange(L, dtype=np.int32), np.array([L], np.int32)
    idx = np.full((L, L), -1, np.int32)
    cnt = np.zeros(L, np.int32)
    for t in range(L):
        c = list(range(max(0, t + 1 - window)))
        idx[t, :len(c)] = c
        cnt[t] = len(c)
    scale = float(np.float32(1.0 / math.sqrt(dqk)))
    o, lse = orc.attention(so, po, sl, 1, window, q, K, None, idx, cnt, scale=scale,
                           v_from_k=True, dv=dv)
    assert o.shape == (S, L, Hq, dv)
    ref, rlse = _sdpa_dense(q.double(), K[0].double(), K[0, :, :, :dv].double().contiguous(),
                            list(range(L)), 1, scale)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, rlse, rtol=1e-12, atol=1e-12)


def test_latent_576_512_single_entry(orc):
    """At the C3 widths (576 / 512): a row that sees one entry returns the
    first 512 channels of that latent row exactly, and two rows with equal
    logits return the mean of the visible rows' first 512 channels."""
    g = torch.Generator().manual_seed(72)
    L, Hq = 6, 3
    K = torch.randn(1, L, 1, 576, generator=g).to(torch.bfloat16)
    q = torch.randn(1, 2, Hq, 576, generator=g).to(torch.bfloat16)
    q[0, 1] = 0
    so, po, sl = np.zeros(2, np.int32), np.array([0, L - 1], np.int32), np.array([L], np.int32)
    o, _ = orc.attention(so, po, sl, 1, L, q, K, None, None, None, scale=576 ** -0.5,
                         v_from_k=True, dv=512)
    first = K[0, 0, 0, :512].double().numpy()
    assert np.array_equal(o[0, 0], np.repeat(first[None], Hq, 0))
    mean = K[0, :, 0, :512].double().mean(0).numpy()
    assert np.allclose(o[0, 1], np.repeat(mean[None], Hq, 0), rtol=1e-14, atol=1e-14)


def test_sink_is_a_zero_valued_entry(orc):
    """A sink logit s joins the normaliser like one more entry whose value row
    is zero ("HySparse2", section 17.1: a learnable per-head sink bias): the
    oracle with sink s equals the oracle without a sink over the same set
    plus an extra entry built so that its logit is exactly s (q[0] = 1,
    k*[0] = s / scale, every other channel zero) and its value row is 0."""
    g = torch.Generator().manual_seed(90)
    L, Hq, d = 20, 3, 8
    scale, s = 0.25, 1.5
    K = torch.randn(1, L + 1, Hq, d, generator=g)
    V = torch.randn(1, L + 1, Hq, d, generator=g)
    q = torch.randn(1, 1, Hq, d, generator=g)
    q[..., 0] = 1.0
    K[0, L] = 0.0
    K[0, L, :, 0] = s / scale
    V[0, L] = 0.0
    so = np.zeros(1, np.int32)
    sl_small, sl_big = np.array([L], np.int32), np.array([L + 1], np.int32)
    a, la = orc.attention(so, np.array([L - 1], np.int32), sl_small, 1, L, q, K, V, None, None,
                          scale=scale, sink=torch.full((1, Hq), s))
    b, lb = orc.attention(so, np.array([L], np.int32), sl_big, 1, L + 1, q, K, V, None, None,
                          scale=scale)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    assert np.allclose(la, lb, rtol=1e-13, atol=1e-15)
    # a sink far below every logit changes nothing
    c, lc = orc.attention(so, np.array([L - 1], np.int32), sl_small, 1, L, q, K, V, None, None,
                          scale=scale, sink=torch.full((1, Hq), -1e30))
    d0, ld = orc.attention(so, np.array([L - 1], np.int32), sl_small, 1, L, q, K, V, None, None,
                           scale=scale)
    assert np.array_equal(c, d0) and np.array_equal(lc, ld)


def test_sink_single_entry_and_empty(orc):
    """One visible entry with logit l and sink s: o = v / (1 + exp(s - l)) and
    lse = log(exp(l) + exp(s)); an empty set gives o = 0 and lse = s."""
    K = torch.tensor([[[[2.0, 0.0]]]])            # [1, 1, 1, 2]
    V = torch.tensor([[[[3.0, -1.0]]]])
    q = torch.tensor([[[[1.0, 5.0]]]])            # logit = scale * 2
    so = np.array([0, -1], np.int32)
    po = np.array([0, 0], np.int32)
    sl = np.array([1], np.int32)
    q2 = torch.cat([q, q], dim=1)
    o, lse = orc.attention(so, po, sl, 1, 1, q2, K, V, None, None, scale=0.5,
                           sink=torch.tensor([[0.25]]))
    lg = 1.0
    assert np.allclose(o[0, 0, 0], np.array([3.0, -1.0]) / (1 + math.exp(0.25 - lg)), rtol=1e-15)
    assert abs(lse[0, 0, 0] - math.log(math.exp(lg) + math.exp(0.25))) < 1e-15
    assert np.all(o[0, 1] == 0) and lse[0, 1, 0] == 0.25


def test_output_gate_closed_forms(orc):
    """The output gate multiplies each channel by 1 / (1 + exp(-g)): g = 0
    halves it exactly, g = ln 3 scales it by 3/4, and a very negative g
    zeroes it; the LSE does not depend on the gate."""
    g_ = torch.Generator().manual_seed(91)
    L, Hq, d = 9, 2, 4
    K = torch.randn(1, L, 1, d, generator=g_)
    V = torch.randn(1, L, 1, d, generator=g_)
    q = torch.randn(1, 1, Hq, d, generator=g_)
    so, po, sl = np.zeros(1, np.int32), np.array([L - 1], np.int32), np.array([L], np.int32)
    base, lb = orc.attention(so, po, sl, 1, L, q, K, V, None, None, scale=0.3)
    gate = torch.zeros(1, 1, Hq, d, dtype=torch.float64)
    gate[..., 1] = math.log(3.0)
    gate[..., 2] = -1e4
    o, lse = orc.attention(so, po, sl, 1, L, q, K, V, None, None, scale=0.3, gate=gate.float())
    assert np.array_equal(o[..., 0], base[..., 0] / 2)
    assert np.allclose(o[..., 1], base[..., 1] * 0.75, rtol=1e-7)
    assert np.all(o[..., 2] == 0.0)
    assert np.array_equal(lse, lb)
