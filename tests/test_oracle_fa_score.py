"""Pins of the oracle's full-attention selection score (no GPU): for every
visible entry, the dense-attention probability each query head gives it,
summed over heads ("HySparse2", appendix A.1: the FA layer selects from its
own attention scores; "Lecture 10", section 5.2: summed over heads).

What fixes the expected values:
  * each head's probabilities over a row's domain sum to one, so a row's
    scores sum to (query sets x heads);
  * one head is a plain softmax of the logits, here from torch.softmax in
    float64 (a library routine) on logits formed by torch;
  * shift invariance: adding one vector to every key moves each head's
    logits by a constant, which leaves softmax unchanged;
  * zero queries give equal logits: every visible entry gets heads / n;
  * a row at position 0 sees one entry, which takes every head's mass;
  * each head's probability equals exp(logit - lse) with the lse of the
    oracle's dense attention (window covering the whole domain).
"""
import math

import numpy as np
import torch


def _rows(t_list, L):
    return (np.zeros(len(t_list), np.int32), np.array(t_list, np.int32),
            np.array([L], np.int32))


def test_rows_sum_to_head_count(orc):
    g = torch.Generator().manual_seed(80)
    L, Hq, Hkv, d, S = 50, 6, 2, 16, 2
    q = torch.randn(S, 5, Hq, d, generator=g)
    K = torch.randn(1, L, Hkv, d, generator=g)
    so, po, sl = _rows([0, 7, 20, 49, 33], L)
    sc = orc.fa_score(so, po, sl, 1, q, K, scale=0.25)
    for r, t in enumerate(po):
        assert np.all(np.isnan(sc[r, t + 1:]))
        assert abs(sc[r, :t + 1].sum() - S * Hq) < 1e-12
        assert np.all(sc[r, :t + 1] > 0)
    assert np.allclose(sc[0, 0], S * Hq, rtol=0, atol=1e-13)


def test_single_head_is_softmax(orc):
    g = torch.Generator().manual_seed(81)
    L, d = 40, 24
    q = torch.randn(1, 3, 1, d, generator=g, dtype=torch.float64).float()
    K = torch.randn(1, L, 1, d, generator=g, dtype=torch.float64).float()
    so, po, sl = _rows([39, 10, 25], L)
    scale = float(np.float32(1 / math.sqrt(d)))
    sc = orc.fa_score(so, po, sl, 1, q, K, scale=scale)
    for r, t in enumerate(po):
        lg = (K[0, :t + 1, 0].double() @ q[0, r, 0].double()) * scale
        p = torch.softmax(lg, 0).numpy()
        assert np.allclose(sc[r, :t + 1], p, rtol=1e-12, atol=1e-15)


def test_shift_invariance_and_gqa(orc):
    g = torch.Generator().manual_seed(82)
    L, Hq, Hkv, d = 30, 8, 4, 8
    # dyadic values keep q . (k + u) = q . k + q . u exact in float64
    q = (torch.randint(-8, 9, (1, 4, Hq, d), generator=g).float() / 8)
    K = (torch.randint(-8, 9, (1, L, Hkv, d), generator=g).float() / 8)
    u = (torch.randint(-8, 9, (1, 1, Hkv, d), generator=g).float() / 8)
    so, po, sl = _rows([29, 3, 17, 0], L)
    a = orc.fa_score(so, po, sl, 1, q, K, scale=0.5)
    b = orc.fa_score(so, po, sl, 1, q, K + u, scale=0.5)
    fin = ~np.isnan(a)
    assert np.allclose(a[fin], b[fin], rtol=1e-12, atol=1e-14)
    # head h reads KV head floor(h * Hkv / Hq): a query that only matches KV
    # head 3 concentrates heads 6 and 7 on the entry built for it
    K2 = torch.zeros(1, L, Hkv, d)
    K2[0, 12, 3] = 4.0
    q2 = torch.zeros(1, 1, Hq, d)
    q2[0, 0, 6:] = 4.0
    s2 = orc.fa_score(*_rows([29], L), 1, q2, K2, scale=1.0)
    # heads 0..5 are uniform (1/30 each); heads 6, 7 put almost all mass on 12
    assert s2[0, 12] > 6 / 30 + 1.99 and abs(s2[0].sum() - Hq) < 1e-12


def test_zero_queries_uniform_and_selection_tie_rule(orc):
    L, Hq = 64, 4
    K = torch.randn(1, L, 1, 8)
    q = torch.zeros(1, 1, Hq, 8)
    so, po, sl = _rows([L - 1], L)
    sc = orc.fa_score(so, po, sl, 1, q, K, scale=1.0)
    assert np.allclose(sc[0], Hq / L, rtol=1e-14)
    # all scores tie: window 8 + top-10 takes the 10 lowest candidates
    idx, cnt = orc.topk_select(so, po, sl, 1, 8, sc, 10)
    assert cnt[0] == 10 and list(idx[0]) == list(range(10))


def test_probabilities_match_dense_attention_lse(orc):
    g = torch.Generator().manual_seed(83)
    L, Hq, Hkv, d = 45, 4, 1, 16
    q = torch.randn(1, 2, Hq, d, generator=g).to(torch.bfloat16)
    K = torch.randn(1, L, Hkv, d, generator=g).to(torch.bfloat16)
    V = torch.randn(1, L, Hkv, d, generator=g).to(torch.bfloat16)
    so, po, sl = _rows([44, 30], L)
    scale = 0.25
    _, lse = orc.attention(so, po, sl, 1, L, q, K, V, None, None, scale=scale)
    sc = orc.fa_score(so, po, sl, 1, q, K, scale=scale)
    for r, t in enumerate(po):
        lg = (K[0, :t + 1, 0].double() @ q[0, r].double().T) * scale  # [n, Hq]
        p = torch.exp(lg - torch.from_numpy(lse[0, r])[None])
        assert np.allclose(sc[r, :t + 1], p.sum(1).numpy(), rtol=1e-12, atol=1e-15)
