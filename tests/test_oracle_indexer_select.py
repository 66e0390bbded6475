"""Pins of the oracle's indexer score, window + top-k selection and block-max
pool (no GPU).

What fixes the expected values:
  * a hand-worked example (tests/golden/indexer_worked.json);
  * invariants of the score (homogeneity, linearity in w, ReLU clipping);
  * a full sort by (score desc, position asc) with Python's ``sorted``;
  * the closed-form budget: count = min(k, available outside the window);
  * the degeneracy and metamorphic properties of the block-max pool.
"""
import json
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(t_list, L):
    so = np.zeros(len(t_list), dtype=np.int32)
    po = np.array(t_list, dtype=np.int32)
    return so, po, np.array([L], dtype=np.int32)


def test_worked_example(orc):
    ex = json.load(open(os.path.join(GOLDEN, "indexer_worked.json")))
    q = torch.tensor([ex["q"]], dtype=torch.float32)          # [1, H, D]
    w = torch.tensor([ex["w"]], dtype=torch.float32)          # [1, H]
    kk = torch.tensor([ex["k"]], dtype=torch.float32)         # [1, L, D]
    L = kk.shape[1]
    so, po, sl = _rows([L - 1], L)
    sc = orc.index_score(so, po, sl, 1, q, w, kk)
    assert np.array_equal(sc[0], np.array(ex["scores"]))
    for case in ex["selections"]:
        t = case["t"]
        so, po, sl = _rows([t], L)
        sc = orc.index_score(so, po, sl, 1, q, w, kk)
        idx, cnt = orc.topk_select(so, po, sl, 1, case["window"], sc, case["k"])
        want = case["idx"]
        assert cnt[0] == len(want), case
        assert list(idx[0, :len(want)]) == want, case
        assert np.all(idx[0, len(want):] == -1)


def test_score_domain_and_stride(orc):
    """Entry e is scored only if stride*(e+1) <= min(t+1, len); others NaN."""
    g = torch.Generator().manual_seed(1)
    L, stride = 37, 4
    q = torch.randn(6, 2, 8, generator=g)
    w = torch.rand(6, 2, generator=g)
    kk = torch.randn(2, L // stride + 2, 8, generator=g)
    so = np.array([0, 0, 1, 1, -1, 0], dtype=np.int32)
    po = np.array([0, 3, 10, 36, 5, 2], dtype=np.int32)
    sl = np.array([L, 30], dtype=np.int32)
    sc = orc.index_score(so, po, sl, stride, q, w, kk)
    for r in range(6):
        vis = 0 if so[r] < 0 else min(po[r] + 1, sl[so[r]])
        n = vis // stride
        assert np.all(np.isfinite(sc[r, :n]))
        assert np.all(np.isnan(sc[r, n:]))


def test_score_invariants(orc):
    g = torch.Generator().manual_seed(2)
    R, H, D, L = 3, 4, 16, 50
    q = torch.randn(R, H, D, generator=g)
    # dyadic weights so that w + w2 is exact in float32
    w = torch.randint(0, 9, (R, H), generator=g).float() / 8
    w2 = torch.randint(0, 9, (R, H), generator=g).float() / 8
    kk = torch.randn(1, L, D, generator=g)
    so, po, sl = np.zeros(R, np.int32), np.array([49, 20, 0], np.int32), np.array([L], np.int32)
    base = orc.index_score(so, po, sl, 1, q, w, kk)
    fin = np.isfinite(base)
    # positive homogeneity in q (x2 is exact)
    assert np.array_equal(orc.index_score(so, po, sl, 1, 2 * q, w, kk)[fin], 2 * base[fin])
    # linearity in w
    s1 = orc.index_score(so, po, sl, 1, q, w2, kk)
    s12 = orc.index_score(so, po, sl, 1, q, w + w2, kk)
    assert np.allclose(s12[fin], (base + s1)[fin], rtol=1e-12, atol=1e-12)
    # a query head that is negatively aligned with every key contributes 0:
    # choose keys with positive first channel and q = -e0 on head 0 only.
    kp = kk.clone()
    kp[..., 0] = kp[..., 0].abs() + 0.1
    kp[..., 1:] = 0
    qn = torch.zeros(1, H, D)
    qn[0, 0, 0] = -1.0
    wn = torch.ones(1, H)
    s = orc.index_score(np.zeros(1, np.int32), np.array([49], np.int32), sl, 1, qn, wn, kp)
    assert np.all(s[0] == 0.0)


def test_score_integer_inputs_exact(orc):
    """Integer inputs give integer scores; check against the same scores
    computed per head with a library matmul in float64."""
    g = torch.Generator().manual_seed(3)
    R, H, D, L = 4, 8, 32, 64
    q = torch.randint(-4, 5, (R, H, D), generator=g).float()
    w = torch.randint(-4, 5, (R, H), generator=g).float()
    kk = torch.randint(-4, 5, (1, L, D), generator=g).float()
    so = np.zeros(R, np.int32)
    po = np.full(R, L - 1, np.int32)
    sl = np.array([L], np.int32)
    sc = orc.index_score(so, po, sl, 1, q, w, kk)
    dots = torch.einsum("rhd,ld->rhl", q.double(), kk[0].double())
    ref = (w.double()[:, :, None] * dots.clamp(min=0)).sum(1).numpy()
    assert np.array_equal(sc, ref)
    assert np.array_equal(sc, np.round(sc))


def _brute_select(scores_row, positions, k):
    order = sorted(zip(positions, scores_row), key=lambda ps: (-ps[1], ps[0]))
    return sorted(p for p, _ in order[:k])


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_full_sort(orc, seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 400))
    R = 8
    window = int(rng.integers(0, 40))
    k = int(rng.integers(1, 120))
    po = rng.integers(0, L, R).astype(np.int32)
    so = np.zeros(R, np.int32)
    sl = np.array([L], np.int32)
    if seed % 2:
        scores = rng.integers(-3, 4, (R, L)).astype(np.float64)  # many ties
        scores[scores == 0] = -0.0 if seed % 3 else 0.0
    else:
        scores = rng.standard_normal((R, L))
    idx, cnt = orc.topk_select(so, po, sl, 1, window, scores, k)
    for r in range(R):
        n = po[r] + 1
        lo = max(0, n - window)
        want = _brute_select(scores[r, :lo], list(range(lo)), k)
        assert cnt[r] == min(k, lo)
        assert list(idx[r, :cnt[r]]) == want
        assert np.all(idx[r, cnt[r]:] == -1)


def test_select_signed_zero_ties(orc):
    """-0 and +0 are the same score: the lower position wins."""
    scores = np.array([[0.0, -0.0, -0.0, 0.0, -1.0]])
    so, po, sl = np.zeros(1, np.int32), np.array([4], np.int32), np.array([5], np.int32)
    idx, cnt = orc.topk_select(so, po, sl, 1, 0, scores, 2)
    assert list(idx[0]) == [0, 1]


def test_select_budget_closed_form(orc):
    """Prefill rows t = 0..n-1 with window w and budget k select
    sum_t min(k, max(0, t+1-w)) positions in total."""
    n, w, k = 600, 16, 96
    so = np.zeros(n, np.int32)
    po = np.arange(n, dtype=np.int32)
    sl = np.array([n], np.int32)
    scores = np.random.default_rng(0).standard_normal((n, n))
    idx, cnt = orc.topk_select(so, po, sl, 1, w, scores, k)
    assert int(cnt.sum()) == sum(min(k, max(0, t + 1 - w)) for t in range(n))
    # invariants: ascending, unique, causal, outside the window
    for t in range(n):
        sel = idx[t, :cnt[t]]
        assert np.all(np.diff(sel) > 0)
        assert np.all(sel <= t - w) if cnt[t] else True


def test_select_candidate_mode(orc):
    rng = np.random.default_rng(7)
    R, P, L = 5, 40, 200
    cand = np.full((R, P), -1, np.int32)
    cc = np.zeros(R, np.int32)
    for r in range(R):
        m = int(rng.integers(0, P + 1))
        cand[r, :m] = np.sort(rng.choice(L, m, replace=False))
        cc[r] = m
    scores = rng.integers(0, 5, (R, P)).astype(np.float64)
    so, po, sl = np.zeros(R, np.int32), np.full(R, L - 1, np.int32), np.array([L], np.int32)
    idx, cnt = orc.topk_select(so, po, sl, 1, 0, scores, 7, cand=cand, cand_count=cc)
    for r in range(R):
        want = _brute_select(scores[r, :cc[r]], list(cand[r, :cc[r]]), 7)
        assert list(idx[r, :cnt[r]]) == want


def _brute_pool(scores_row, n, block, max_blocks):
    blocks = []
    for j in range((n + block - 1) // block):
        mem = list(range(j * block, min(n, (j + 1) * block)))
        blocks.append((j, max(scores_row[s] for s in mem), mem))
    keep = sorted(blocks, key=lambda b: (-b[1], b[0]))[:max_blocks]
    return sorted(s for b in keep for s in b[2])


@pytest.mark.parametrize("seed", range(4))
def test_block_pool_matches_brute_force(orc, seed):
    rng = np.random.default_rng(100 + seed)
    L, R, block, mb = 333, 6, 8, int(rng.integers(1, 30))
    po = rng.integers(0, L, R).astype(np.int32)
    so, sl = np.zeros(R, np.int32), np.array([L], np.int32)
    scores = rng.integers(0, 6, (R, L)).astype(np.float64) if seed % 2 else rng.standard_normal((R, L))
    idx, cnt, pool, pc = orc.topk_select(so, po, sl, 1, 0, scores, 4, block=block, max_blocks=mb)
    for r in range(R):
        want = _brute_pool(scores[r], po[r] + 1, block, mb)
        assert list(pool[r, :pc[r]]) == want
        assert np.all(pool[r, pc[r]:] == -1)


def test_block_pool_degenerate_is_whole_domain(orc):
    rng = np.random.default_rng(11)
    L, R = 301, 4
    po = np.array([0, 7, 150, 300], np.int32)
    so, sl = np.zeros(R, np.int32), np.array([L], np.int32)
    scores = rng.standard_normal((R, L))
    _, _, pool, pc = orc.topk_select(so, po, sl, 1, 0, scores, 1, block=8, max_blocks=1000)
    for r in range(R):
        assert list(pool[r, :pc[r]]) == list(range(po[r] + 1))


def test_reindex_with_own_query_returns_full_topk(orc):
    """Metamorphic pin: rescoring only the block-max pool with the Full
    layer's own query, then selecting top-k inside it, gives exactly the
    Full layer's top-k (the pool keeps at least as many blocks as k)."""
    g = torch.Generator().manual_seed(12)
    R, H, D, L, k = 6, 4, 16, 700, 24
    for integer in (False, True):
        if integer:
            q = torch.randint(-4, 5, (R, H, D), generator=g).float()
            w = torch.randint(0, 5, (R, H), generator=g).float()
            kk = torch.randint(-4, 5, (1, L, D), generator=g).float()
        else:
            q = torch.randn(R, H, D, generator=g)
            w = torch.rand(R, H, generator=g)
            kk = torch.randn(1, L, D, generator=g)
        so = np.zeros(R, np.int32)
        po = np.array([L - 1, 500, 300, 100, 40, 5], np.int32)
        sl = np.array([L], np.int32)
        sc = orc.index_score(so, po, sl, 1, q, w, kk)
        idx, cnt, pool, pc = orc.topk_select(so, po, sl, 1, 0, sc, k, block=8, max_blocks=k)
        rs = orc.index_score(so, po, sl, 1, q, w, kk, cand=pool, cand_count=pc)
        ridx, rcnt = orc.topk_select(so, po, sl, 1, 0, rs, k, cand=pool, cand_count=pc)
        assert np.array_equal(cnt, rcnt)
        for r in range(R):
            assert set(idx[r, :cnt[r]]) <= set(pool[r, :pc[r]])
        assert np.array_equal(idx, ridx)


@pytest.mark.parametrize("window", [5, 64, 200])
def test_block_pool_with_window_is_block_selection(orc, window):
    """With a forced window the blocks range over the candidates only (the
    visible positions before the window): the pool equals the brute-force
    block choice over [0, win_lo), never holds a window position, and with
    max_blocks covering every block it is exactly [0, win_lo).  This is the
    first-generation HySparse block selection ("HySparse2", appendix A.1: 16
    blocks of 64 tokens next to a window of 128) in the index format; with
    max_blocks >= k the token top-k lies inside it."""
    rng = np.random.default_rng(300 + window)
    L, R, block, mb = 700, 5, 64, 4
    po = np.array([699, 400, 250, 64, 3], np.int32)
    so, sl = np.zeros(R, np.int32), np.array([L], np.int32)
    scores = rng.integers(0, 9, (R, L)).astype(np.float64)
    idx, cnt, pool, pc = orc.topk_select(so, po, sl, 1, window, scores, mb, block=block,
                                         max_blocks=mb)
    _, _, full, fc = orc.topk_select(so, po, sl, 1, window, scores, 1, block=block,
                                     max_blocks=1000)
    for r in range(R):
        win_lo = max(0, po[r] + 1 - window)
        want = _brute_pool(scores[r], win_lo, block, mb)
        assert list(pool[r, :pc[r]]) == want
        assert np.all(pool[r, pc[r]:] == -1) and (pc[r] == 0 or pool[r, pc[r] - 1] < win_lo)
        assert list(full[r, :fc[r]]) == list(range(win_lo))
        assert set(idx[r, :cnt[r]]) <= set(pool[r, :pc[r]])
