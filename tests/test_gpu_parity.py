"""GPU parity: every entry point of the HIP library against the fp64 oracle on
seeded inputs of each workload's shape family, at oracle-friendly sizes that
still span several tiles, pages and splits, with ragged and degenerate rows.

Index sets are bit-exact on integer-valued inputs; on float inputs only
boundary swaps within the fp32 error bound are allowed.  Attention is checked
given identical (oracle-chosen) indices: max-abs 1e-2 / rel-L2 5e-3 for bf16
and FP4 (after the same exact dequantisation), 1e-5 / 1e-6 for fp32.
"""
import numpy as np
import pytest
import torch

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import index_reuse_amd

    index_reuse_amd.load()
    return "cuda"


def _cases():
    hs2 = synth.HYSPARSE2.replace(n_seqs=7, seq_lens_override=(2500, 1151, 1152, 1153, 100, 1, 1280))
    csa = synth.CSA.replace(n_seqs=4, seq_len=8192, tail_variant=True)
    csa2 = synth.CSA2.replace(n_seqs=2, seq_lens_override=(20000, 16389))
    tiny = synth.TINY
    return {
        "tiny": (tiny, False),
        "tiny_int": (tiny, True),
        "hysparse2": (hs2, False),
        "hysparse2_int": (hs2, True),
        "csa": (csa, False),
        "csa_int": (csa, True),
        "csa2": (csa2, False),
        "csa2_int": (csa2, True),
    }


CASES = _cases()
DSA_ROWS = [0, 1, 2, 63, 64, 100, 2046, 2047, 2048, 2049, 3000, 4095]


def _problem(name):
    wl, integer = CASES[name]
    return wl, integer, synth.make_problem(wl, device="cpu", integer=integer)


def _step(prob, dev):
    from index_reuse_amd.pipeline import Step

    p = H.move(prob, dev)
    return p, Step(p)


def _flush(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_index_and_select(name, dev):
    wl, integer, prob = _problem(name)
    _flush("case %s R=%d" % (name, prob.n_rows))
    p, step = _step(prob, dev)
    step.run_index()
    torch.cuda.synchronize()
    sc = H.oracle_scores(prob, 0)
    g = step.scores[0].cpu().double().numpy()
    valid = ~np.isnan(sc)
    tau = None if integer else H.fp32_score_bound(prob, 0)
    if integer:
        assert np.array_equal(g[valid], sc[valid])
    else:
        err = np.abs(g - np.nan_to_num(sc))
        assert np.all(err[valid] <= np.broadcast_to(tau[:, None], sc.shape)[valid])
    if not wl.block:
        idx, cnt = H.oracle_select(prob, sc, wl.k)
        H.check_indices(step.idx[0].cpu(), step.count[0].cpu(), idx, cnt, sc, tau,
                        win_lo=H.win_lo(prob))
        return
    idx, cnt, pool, pc = H.oracle_select(prob, sc, wl.k, block=wl.block, max_blocks=wl.max_blocks)
    H.check_indices(step.idx[0].cpu(), step.count[0].cpu(), idx, cnt, sc, tau,
                    win_lo=H.win_lo(prob))
    gpool, gpc = step.pool.cpu().numpy(), step.pool_count.cpu().numpy()
    if integer:
        assert np.array_equal(gpc, pc)
        assert np.array_equal(gpool, pool)
    same = [r for r in range(prob.n_rows) if np.array_equal(gpool[r], pool[r])]
    assert len(same) >= (prob.n_rows if integer else 1)
    # Reindex over the (identical) pool with the second query
    rs = H.oracle_scores(prob, 1, cand=pool, cand_count=pc)
    gr = step.scores[1].cpu().double().numpy()
    for r in same:
        v = ~np.isnan(rs[r])
        if integer:
            assert np.array_equal(gr[r, v], rs[r, v])
    ridx, rcnt = H.oracle_select(prob, rs, wl.k, cand=pool, cand_count=pc)
    tau1 = None if integer else H.fp32_score_bound(prob, 1)
    H.check_indices(step.idx[1].cpu(), step.count[1].cpu(), ridx, rcnt, rs, tau1, rows=same,
                    positions=pool, win_lo=H.win_lo(prob))


@pytest.mark.parametrize("name", list(CASES))
def test_attention_given_oracle_indices(name, dev):
    wl, integer, prob = _problem(name)
    _flush("case %s R=%d" % (name, prob.n_rows))
    p, step = _step(prob, dev)
    sc = H.oracle_scores(prob, 0)
    if wl.block:
        idx, cnt, pool, pc = H.oracle_select(prob, sc, wl.k, block=wl.block,
                                             max_blocks=wl.max_blocks)
        rs = H.oracle_scores(prob, 1, cand=pool, cand_count=pc)
        ridx, rcnt = H.oracle_select(prob, rs, wl.k, cand=pool, cand_count=pc)
        idxs, cnts = [idx, ridx], [cnt, rcnt]
    else:
        idx, cnt = H.oracle_select(prob, sc, wl.k)
        idxs, cnts = [idx], [cnt]
    tidx = [torch.from_numpy(np.ascontiguousarray(i)).to(dev) for i in idxs]
    tcnt = [torch.from_numpy(np.ascontiguousarray(c)).to(dev) for c in cnts]
    step.run_attention(idx=tidx, count=tcnt)
    torch.cuda.synchronize()
    for c in range(len(prob.q)):
        o_ref, l_ref = H.oracle_attention(prob, c, idxs[c], cnts[c])
        H.check_outputs(step.o[c], o_ref, step.lse[c], l_ref, wl.attn_dtype,
                        what="%s call %d" % (name, c))


# Decode-indexer layouts: groups of 64 entries in pages of 64, 128 or 256
# (at offsets inside a page), pages of 32 (per-tile page reads), 128- and
# 256-byte bf16 rows, FP8 rows, and contiguous caches; ragged lengths.
INDEX_LAYOUTS = {
    "bf16_d64_page128": dict(page_size=128),
    "bf16_d128_page256": dict(idx_dim=128, idx_heads=32, page_size=256),
    "bf16_d64_page32": dict(page_size=32),
    "fp8_d128_h64_page64": dict(idx_dtype=torch.float8_e4m3fn, idx_dim=128, idx_heads=64),
    "bf16_d64_contiguous": dict(page_size=0),
}


@pytest.mark.parametrize("layout", list(INDEX_LAYOUTS))
@pytest.mark.parametrize("integer", [True, False])
def test_decode_indexer_layouts(layout, integer, dev):
    wl = synth.HYSPARSE2.replace(n_seqs=4, seq_lens_override=(3000, 1151, 130, 2049),
                                 **INDEX_LAYOUTS[layout])
    prob = synth.make_problem(wl, device="cpu", integer=integer)
    _flush("case %s integer=%s" % (layout, integer))
    p, step = _step(prob, dev)
    step.run_index()
    torch.cuda.synchronize()
    sc = H.oracle_scores(prob, 0)
    g = step.scores[0].cpu().double().numpy()
    valid = ~np.isnan(sc)
    if integer:
        assert np.array_equal(g[valid], sc[valid])
    else:
        tau = H.fp32_score_bound(prob, 0)
        err = np.abs(g - np.nan_to_num(sc))
        assert np.all(err[valid] <= np.broadcast_to(tau[:, None], sc.shape)[valid])


# Window-first attention ranges: a window that is not a whole number of
# steps (rows with fewer visible entries than the window, between one step
# and the window, and longer), and a single row, which the launch splits
# over many workgroups (only the first split opens with the window step).
WINDOW_CASES = {
    "window200": dict(window=200, n_seqs=4, seq_lens_override=(3000, 150, 90, 1500)),
    "single_row_split": dict(n_seqs=1, seq_lens_override=(5000,)),
}


@pytest.mark.parametrize("case", list(WINDOW_CASES))
def test_attention_window_ranges(case, dev):
    wl = synth.HYSPARSE2.replace(**WINDOW_CASES[case])
    prob = synth.make_problem(wl, device="cpu")
    _flush("case %s" % case)
    p, step = _step(prob, dev)
    sc = H.oracle_scores(prob, 0)
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    step.run_attention(idx=[torch.from_numpy(idx).to(dev)], count=[torch.from_numpy(cnt).to(dev)])
    torch.cuda.synchronize()
    for c in range(len(prob.q)):
        o_ref, l_ref = H.oracle_attention(prob, c, idx, cnt)
        H.check_outputs(step.o[c], o_ref, step.lse[c], l_ref, wl.attn_dtype,
                        what="%s call %d" % (case, c))


ATTN_SHAPES = {
    # 10 query sets x 8 heads per KV head: 80 rows, two row groups per KV head
    "sep128_q10": dict(n_qsets=10),
    # 16 query heads per KV head, 3 sets
    "sep128_g16": dict(hq=64, hkv=4, n_qsets=3),
    # one 128-wide row serving as K and V
    "shared128": dict(kv_mode="shared", hq=32, hkv=2, n_qsets=2),
    # separate K and V rows of 256 channels
    "sep256": dict(dqk=256, dv=256, hq=16, hkv=2, n_qsets=2),
    # 576-wide latent rows (V = first 512): 16 query rows per KV head (one
    # row tile per wave), 2 x 64 rows (two 64-row groups), and 80 rows (a
    # partial second group)
    "latent_h16": dict(dqk=576, dv=512, kv_mode="shared", hq=16, hkv=1, n_qsets=1),
    "latent_h64_q2": dict(dqk=576, dv=512, kv_mode="shared", hq=64, hkv=1, n_qsets=2),
    "latent_h80": dict(dqk=576, dv=512, kv_mode="shared", hq=80, hkv=1, n_qsets=1),
}


@pytest.mark.parametrize("shape", list(ATTN_SHAPES))
def test_attention_shapes(shape, dev):
    """Gather attention for other head / width / query-set layouts (the kernel
    picks a different work shape for each) against the oracle, given oracle
    indices."""
    wl = synth.HYSPARSE2.replace(n_seqs=3, seq_lens_override=(3000, 777, 1500),
                                 **ATTN_SHAPES[shape])
    prob = synth.make_problem(wl, device="cpu")
    _flush("case %s" % shape)
    p, step = _step(prob, dev)
    sc = H.oracle_scores(prob, 0)
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    step.run_attention(idx=[torch.from_numpy(idx).to(dev)], count=[torch.from_numpy(cnt).to(dev)])
    torch.cuda.synchronize()
    o_ref, l_ref = H.oracle_attention(prob, 0, idx, cnt)
    H.check_outputs(step.o[0], o_ref, step.lse[0], l_ref, torch.bfloat16, what=shape)


@pytest.mark.parametrize("shape,gain", [("sep128", 8.0), ("sep128", 40.0), ("dsa576", 40.0)])
def test_attention_peaked_logits(shape, gain, dev):
    """Queries scaled by `gain` spread the logits of a row over a wide range,
    so the row's largest logit often lies in a tile far after the first one
    (beyond 2^64 in the exp2 domain at gain 40, which makes the kernel re-run
    the range with the true maximum as reference)."""
    if shape == "sep128":
        wl = synth.HYSPARSE2.replace(n_seqs=3, seq_lens_override=(3000, 777, 1500))
        prob = synth.make_problem(wl, device="cpu")
    else:
        wl = synth.DSA.replace(seq_len=4096)
        prob = synth.make_problem(wl, device="cpu", rows=DSA_ROWS)
    prob.q[0] = (prob.q[0].float() * gain).to(prob.q[0].dtype)
    _flush("case %s gain %g" % (shape, gain))
    p, step = _step(prob, dev)
    # fp32 outputs: a peaked row's output is close to one V row, whose
    # magnitude can reach 4, where bf16 output rounding alone is 1.6e-2
    step.o[0] = torch.empty(step.o[0].shape, dtype=torch.float32, device=dev)
    sc = H.oracle_scores(prob, 0)
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    step.run_attention(idx=[torch.from_numpy(idx).to(dev)], count=[torch.from_numpy(cnt).to(dev)])
    torch.cuda.synchronize()
    o_ref, l_ref = H.oracle_attention(prob, 0, idx, cnt)
    H.check_outputs(step.o[0], o_ref, step.lse[0], l_ref, torch.bfloat16,
                    what="%s gain %g" % (shape, gain))


@pytest.mark.parametrize("dqk", [576, 512])
def test_attention_leading_padding(dqk, dev):
    """Index lists whose first entries are padding (-1 inside the count, which
    the format allows): the first tiles of a row hold no entry, so the
    reference max of the softmax comes from a later tile; 64 query heads per
    KV head, so the latent kernel with split waves runs."""
    # 24 decode rows: several tiles per split, so the padding covers whole
    # tiles at the start of a split, part of one, or whole splits
    lens = (3000, 1500, 777, 2100) * 6
    wl = synth.HYSPARSE2.replace(n_seqs=len(lens), seq_lens_override=lens, window=0, dqk=dqk,
                                 dv=512, kv_mode="shared", hq=64, hkv=1, n_qsets=1)
    prob = synth.make_problem(wl, device="cpu")
    _flush("case leading padding dqk %d" % dqk)
    p, step = _step(prob, dev)
    sc = H.oracle_scores(prob, 0)
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    idx = idx.copy()
    lead = (40, 70, 100, 500, 0)
    for r in range(idx.shape[0]):
        m = min(lead[r % len(lead)], int(cnt[r]))
        idx[r, :m] = -1
    step.run_attention(idx=[torch.from_numpy(idx).to(dev)], count=[torch.from_numpy(cnt).to(dev)])
    torch.cuda.synchronize()
    o_ref, l_ref = H.oracle_attention(prob, 0, idx, cnt)
    H.check_outputs(step.o[0], o_ref, step.lse[0], l_ref, torch.bfloat16,
                    what="leading padding %d" % dqk)


def test_dsa_rows_fp8_latent(dev):
    """DSA-shaped prefill rows (FP8 indexer 64x128, top-2048, latent 576 with
    V = first 512, 128 heads) on a 4096-token sequence; rows straddle the
    point where the budget stops covering the whole causal prefix."""
    for integer in (True, False):
        wl = synth.DSA.replace(seq_len=4096)
        prob = synth.make_problem(wl, device="cpu", integer=integer, rows=DSA_ROWS)
        _flush("case dsa integer=%s" % integer)
        p, step = _step(prob, dev)
        step.run_index()
        torch.cuda.synchronize()
        sc = H.oracle_scores(prob, 0)
        g = step.scores[0].cpu().double().numpy()
        valid = ~np.isnan(sc)
        if integer:
            assert np.array_equal(g[valid], sc[valid])
            tau = None
        else:
            tau = H.fp32_score_bound(prob, 0)
        idx, cnt = H.oracle_select(prob, sc, wl.k)
        assert list(cnt) == [min(2048, t + 1) for t in DSA_ROWS]
        H.check_indices(step.idx[0].cpu(), step.count[0].cpu(), idx, cnt, sc, tau,
                        win_lo=H.win_lo(prob))
        step.run_attention(idx=[torch.from_numpy(idx).to(dev)], count=[torch.from_numpy(cnt).to(dev)])
        torch.cuda.synchronize()
        o_ref, l_ref = H.oracle_attention(prob, 0, idx, cnt)
        H.check_outputs(step.o[0], o_ref, step.lse[0], l_ref, torch.bfloat16, what="dsa")


def test_prefill_indexer_blocks(dev):
    """The prefill (row-block GEMM) indexer: blocks of consecutive rows of one
    sequence, blocks mixing two sequences, and padding rows, with the FP8
    64x128 indexer; exact on integer inputs, within the fp32 bound on
    N(0,1) inputs."""
    import dataclasses

    from index_reuse_amd import Cache, Rows, index_score

    wl = synth.DSA.replace(n_seqs=2, seq_lens_override=(3000, 1500))
    pos0 = list(range(0, 40)) + list(range(2030, 2070)) + [2999]
    rows = [(0, t) for t in pos0] + [(1, t) for t in range(1480, 1500)]
    rows += [(0, 5), (1, 7), (0, 2500), (1, 1499), (-1, -1), (0, 1024)] * 3
    for integer in (True, False):
        base = synth.make_problem(wl, device="cpu", integer=integer, rows=[0])
        R = len(rows)
        so = torch.tensor([b for b, _ in rows], dtype=torch.int32)
        po = torch.tensor([t for _, t in rows], dtype=torch.int32)
        draw = synth.small_ints if integer else synth.normal
        q = draw((R, wl.idx_heads, wl.idx_dim), seed=4242, dtype=wl.idx_dtype)
        if integer:
            w = synth.small_ints((R, wl.idx_heads), seed=4243, lo=0)
        else:
            w = synth.uniform01((R, wl.idx_heads), seed=4243)
        prob = dataclasses.replace(base, seq_of_row=so, pos_of_row=po, idx_q=[q], idx_w=[w])
        _flush("case prefill indexer integer=%s R=%d" % (integer, R))
        p = H.move(prob, dev)
        S = wl.n_entries_cap
        scores = torch.full((R, S), float("nan"), dtype=torch.float32, device=dev)
        rr = Rows(p.seq_of_row, p.pos_of_row, p.seq_len, wl.stride, wl.window)
        kc = Cache(p.kidx.pool, p.kidx.block_table, 1, wl.idx_dim)
        index_score(rr, p.idx_q[0], p.idx_w[0], kc, scores=scores)
        torch.cuda.synchronize()
        sc = H.oracle_scores(prob, 0)
        g = scores.cpu().double().numpy()
        valid = ~np.isnan(sc)
        assert not np.isnan(g[valid]).any()
        if integer:
            assert np.array_equal(g[valid], sc[valid])
        else:
            tau = H.fp32_score_bound(prob, 0)
            err = np.abs(g - np.nan_to_num(sc))
            assert np.all(err[valid] <= np.broadcast_to(tau[:, None], sc.shape)[valid])


def test_select_exact_on_given_scores(dev):
    """Selection alone on generated scores with heavy ties and signed zeros
    (token, candidate and pool modes) is bit-exact."""
    from index_reuse_amd import Rows, topk_select

    import oracle

    R, S = 24, 5000
    scores = synth.small_ints((R, S), seed=77, lo=-3, hi=3)
    scores[scores == 0] = -0.0
    scores[:, ::7] = 0.0
    scores[3] = 1.0  # one row of all-equal scores
    so = torch.zeros(R, dtype=torch.int32)
    po = torch.tensor([S - 1 - 37 * r for r in range(R)], dtype=torch.int32)
    sl = torch.tensor([S], dtype=torch.int32)
    for window, k in ((0, 1), (16, 700), (100, 4096), (3, 4999)):
        rows = Rows(so.to(dev), po.to(dev), sl.to(dev), 1, window)
        gi, gc, gp, gpc = topk_select(rows, scores.to(dev), k, block=8, max_blocks=100)
        oi, oc, op, opc = oracle.topk_select(so, po, sl, 1, window, scores.double().numpy(), k,
                                             block=8, max_blocks=100)
        torch.cuda.synchronize()
        assert np.array_equal(gc.cpu().numpy(), oc)
        assert np.array_equal(gi.cpu().numpy(), oi)
        assert np.array_equal(gpc.cpu().numpy(), opc)
        assert np.array_equal(gp.cpu().numpy(), op)
    # candidate mode
    P = 1500
    cand = torch.full((R, P), -1, dtype=torch.int32)
    cc = torch.zeros(R, dtype=torch.int32)
    g = torch.Generator().manual_seed(5)
    for r in range(R):
        m = int(torch.randint(0, P + 1, (1,), generator=g))
        cand[r, :m] = torch.randperm(S, generator=g)[:m].sort().values.to(torch.int32)
        cc[r] = m
    cs = scores[:, :P].contiguous()
    rows = Rows(so.to(dev), po.to(dev), sl.to(dev), 1, 10)
    gi, gc = topk_select(rows, cs.to(dev), 300, cand=cand.to(dev), cand_count=cc.to(dev))
    oi, oc = oracle.topk_select(so, po, sl, 1, 10, cs.double().numpy(), 300, cand=cand,
                                cand_count=cc)
    torch.cuda.synchronize()
    assert np.array_equal(gc.cpu().numpy(), oc)
    assert np.array_equal(gi.cpu().numpy(), oi)


def test_select_crowded_threshold_bin(dev):
    """Rows whose threshold falls in a crowded top-12-bit key bin: thousands
    of distinct keys (more than the per-row member list holds), thousands of
    exact ties at the threshold, and both at once.  Token and pool selection
    stay bit-exact against the oracle."""
    from index_reuse_amd import Rows, topk_select

    import oracle

    S = 20000
    g = torch.Generator().manual_seed(11)
    ulp = 2.0 ** -23
    rows = []
    # distinct values in [1, 1.125): one level-1 bin holds all of them
    perm = torch.randperm(S, generator=g).double()
    rows.append(1.0 + perm * 32 * ulp)
    # 6000 ties at 1.5 straddling the threshold, larger and smaller values around
    r = torch.rand(S, generator=g).double()
    idx = torch.randperm(S, generator=g)
    r[idx[:6000]] = 1.5
    r[idx[6000:8000]] = 3.0
    rows.append(r)
    # 3000 distinct values in one bin, each repeated about 7 times
    rows.append(1.0 + (torch.randperm(S, generator=g) % 3000).double() * 64 * ulp)
    # mostly one bin, with signed zeros and a few negatives
    r = 1.0 + torch.randperm(S, generator=g).double() * 16 * ulp
    r[idx[:500]] = -0.0
    r[idx[500:700]] = 0.0
    r[idx[700:900]] = -2.0
    rows.append(r)
    scores = torch.stack(rows).float()
    R = scores.shape[0]
    so = torch.zeros(R, dtype=torch.int32)
    po = torch.full((R,), S - 1, dtype=torch.int32)
    sl = torch.tensor([S], dtype=torch.int32)
    for window, k, mb in ((0, 5000, 1000), (0, 4000, 2048), (50, 12000, 600)):
        rr = Rows(so.to(dev), po.to(dev), sl.to(dev), 1, window)
        gi, gc, gp, gpc = topk_select(rr, scores.to(dev), k, block=8, max_blocks=mb)
        oi, oc, op, opc = oracle.topk_select(so, po, sl, 1, window, scores.double().numpy(), k,
                                             block=8, max_blocks=mb)
        torch.cuda.synchronize()
        assert np.array_equal(gc.cpu().numpy(), oc)
        assert np.array_equal(gi.cpu().numpy(), oi), (window, k)
        assert np.array_equal(gpc.cpu().numpy(), opc)
        assert np.array_equal(gp.cpu().numpy(), op), (window, k, mb)


def test_select_many_rows(dev):
    """Selection over many long rows (the prefill regime, where each
    workgroup takes a larger chunk): 2048 rows of up to 16384 candidates with
    integer ties and signed zeros, bit-exact against the oracle."""
    from index_reuse_amd import Rows, topk_select

    import oracle

    R, S = 2048, 16384
    scores = synth.small_ints((R, S), seed=99, lo=-20, hi=20)
    scores[scores == 0] = -0.0
    scores[7] = 2.0  # a row of ties
    so = torch.zeros(R, dtype=torch.int32)
    po = torch.tensor([S - 1 - 5 * r for r in range(R)], dtype=torch.int32)
    sl = torch.tensor([S], dtype=torch.int32)
    for window, k in ((0, 1000), (64, 3000)):
        rows = Rows(so.to(dev), po.to(dev), sl.to(dev), 1, window)
        gi, gc = topk_select(rows, scores.to(dev), k)
        oi, oc = oracle.topk_select(so, po, sl, 1, window, scores.double().numpy(), k)
        torch.cuda.synchronize()
        assert np.array_equal(gc.cpu().numpy(), oc)
        assert np.array_equal(gi.cpu().numpy(), oi), (window, k)


def test_select_few_long_rows(dev):
    """The decode regime: a few rows of 16385 to 32768 candidates with
    integer ties (one tie block of 400 at the top), a row of all-equal
    scores, a padding row, and windows; bit-exact against the oracle."""
    from index_reuse_amd import Rows, topk_select

    import oracle

    R, S = 9, 32768
    scores = synth.small_ints((R, S), seed=31, lo=-40, hi=40)
    scores[scores == 0] = -0.0
    scores[2] = 5.0                      # all ties
    scores[3, 8000:8400] = 100.0         # a tie block across the first part boundary
    so = torch.zeros(R, dtype=torch.int32)
    so[8] = -1                           # a padding row
    po = torch.tensor([S - 1, S - 2, S - 1, 16384, 20000, S - 1, 17000, 30000, S - 1],
                      dtype=torch.int32)
    sl = torch.tensor([S], dtype=torch.int32)
    for window, k in ((0, 1024), (128, 2048), (7, 100)):
        rows = Rows(so.to(dev), po.to(dev), sl.to(dev), 1, window)
        gi, gc = topk_select(rows, scores.to(dev), k)
        oi, oc = oracle.topk_select(so, po, sl, 1, window, scores.double().numpy(), k)
        torch.cuda.synchronize()
        assert np.array_equal(gc.cpu().numpy(), oc), (window, k)
        assert np.array_equal(gi.cpu().numpy(), oi), (window, k)


def test_select_long_rows_chunked(dev):
    """Rows longer than one workgroup holds in registers (65536 keys) take
    the chunk-parallel path: token selection over 100000-entry rows with a
    wide tie at the threshold, next to the block pool of the same rows,
    bit-exact."""
    from index_reuse_amd import Rows, topk_select

    import oracle

    R, S = 3, 100000
    scores = synth.small_ints((R, S), seed=123, lo=-50, hi=50)
    scores[scores == 0] = -0.0
    scores[1, 5000:60000] = 7.0  # a wide tie straddling the threshold
    so = torch.zeros(R, dtype=torch.int32)
    po = torch.tensor([S - 1, S - 2, S - 1000], dtype=torch.int32)
    sl = torch.tensor([S], dtype=torch.int32)
    for window, k, mb in ((0, 3000, 2000), (40, 20000, 1000)):
        rows = Rows(so.to(dev), po.to(dev), sl.to(dev), 1, window)
        gi, gc, gp, gpc = topk_select(rows, scores.to(dev), k, block=8, max_blocks=mb)
        oi, oc, op, opc = oracle.topk_select(so, po, sl, 1, window, scores.double().numpy(), k,
                                             block=8, max_blocks=mb)
        torch.cuda.synchronize()
        assert np.array_equal(gc.cpu().numpy(), oc)
        assert np.array_equal(gi.cpu().numpy(), oi), (window, k)
        assert np.array_equal(gpc.cpu().numpy(), opc)
        assert np.array_equal(gp.cpu().numpy(), op), (window, k, mb)


@pytest.mark.parametrize("name", ["hysparse2", "csa2"])
def test_graph_replay_matches_eager(name, dev):
    """A whole step captured as one HIP graph (as the throughput benchmark
    replays it) gives bit-identical outputs on every replay, with eager work
    and synchronisation between replays and the outputs cleared before each."""
    wl, _ = CASES[name]
    _flush("case graph %s" % name)
    p, step = _step(synth.make_problem(wl, device="cpu"), dev)
    p2, other = _step(synth.make_problem(wl, device="cpu", seed_base=777), dev)
    calls = step.prepare()
    others = other.prepare()
    stream = torch.cuda.current_stream().cuda_stream
    outs = lambda st: [t for t in (st.scores + st.idx + st.count + st.o + st.lse
                                   + [st.pool, st.pool_count]) if t is not None]
    for t in outs(step):  # entries no call writes stay zero on both sides
        t.zero_()
    for _, c in calls:
        c(stream)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs(step)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for _, c in calls:
            c(cs)
    for rep in range(3):
        for t in outs(step):
            t.zero_()
        for _, c in others:  # the program's own eager work between replays
            c(stream)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(step), ref):
            assert torch.equal(a, b), (name, rep)


@pytest.mark.parametrize("name", ["hysparse2", "csa2"])
def test_steps_in_flight_match_serial(name, dev):
    """Independent steps issued on four streams of one HIP graph (the
    benchmark's steps in flight) give the outputs each step gives alone: no
    workspace or other state is shared between the steps."""
    wl, _ = CASES[name]
    _flush("case in flight %s" % name)
    n = 4
    steps = [_step(synth.make_problem(wl, device="cpu", seed_base=900 + 50 * i), dev)[1]
             for i in range(n)]
    outs = lambda st: [t for t in (st.scores + st.idx + st.count + st.o + st.lse
                                   + [st.pool, st.pool_count]) if t is not None]
    stream = torch.cuda.current_stream().cuda_stream
    refs = []
    for st in steps:
        for t in outs(st):
            t.zero_()
        for _, c in st.prepare():
            c(stream)
        torch.cuda.synchronize()
        refs.append([t.clone() for t in outs(st)])
    g = torch.cuda.CUDAGraph()
    sides = [torch.cuda.Stream() for _ in range(n - 1)]
    with torch.cuda.graph(g):
        main = torch.cuda.current_stream()
        for sd in sides:
            sd.wait_stream(main)
        sts = [main] + sides
        for i in range(2 * n):  # each step twice, step j always on stream j
            st_ = sts[i % n]
            with torch.cuda.stream(st_):
                for _, c in steps[i % n].prepare():
                    c(st_.cuda_stream)
        for sd in sides:
            main.wait_stream(sd)
    for rep in range(2):
        for st in steps:
            for t in outs(st):
                t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, st in enumerate(steps):
            for a, b in zip(outs(st), refs[k]):
                assert torch.equal(a, b), (name, rep, k)


def test_deterministic_and_reuse(dev):
    """Two runs are bitwise identical; one fused call over all query sets
    equals one call per set (index reuse changes nothing numerically)."""
    from index_reuse_amd import attn_gather_fwd

    wl, integer, prob = _problem("hysparse2")
    p, step = _step(prob, dev)
    step.run()
    torch.cuda.synchronize()
    first = [t.clone() for t in step.o] + [step.idx[0].clone()]
    step.run()
    torch.cuda.synchronize()
    for a, b in zip(first, [t for t in step.o] + [step.idx[0]]):
        assert torch.equal(a, b)
    q = p.q[0]
    for s in range(q.shape[0]):
        o1, l1 = attn_gather_fwd(step.rows, q[s:s + 1].contiguous(), step.k, step.v,
                                 idx=step.idx[0], count=step.count[0], scale=step.scale)
        torch.cuda.synchronize()
        ref = step.o[0][s:s + 1].float()
        assert (o1.float() - ref).abs().max().item() <= 1e-2


def test_padding_rows_and_empty(dev):
    """Padding rows (negative sequence) and rows whose window covers their
    whole domain give count 0, o = 0 and lse = -inf."""
    wl = synth.HYSPARSE2.replace(n_seqs=2, seq_lens_override=(300, 50))
    prob = synth.make_problem(wl, device="cpu")
    prob.seq_of_row = torch.tensor([0, -1, 1, 0], dtype=torch.int32)
    prob.pos_of_row = torch.tensor([299, 10, 49, -1], dtype=torch.int32)
    for layer in range(len(prob.idx_q)):
        prob.idx_q[layer] = torch.cat([prob.idx_q[layer]] * 2)
        prob.idx_w[layer] = torch.cat([prob.idx_w[layer]] * 2)
    prob.q = [torch.cat([q, q], dim=1) for q in prob.q]
    p, step = _step(prob, dev)
    step.run()
    torch.cuda.synchronize()
    cnt = step.count[0].cpu().tolist()
    assert cnt == [172, 0, 0, 0]
    o = step.o[0].float().cpu()
    lse = step.lse[0].cpu()
    for r in (1, 3):
        assert torch.all(o[:, r] == 0) and torch.all(torch.isneginf(lse[:, r]))
    sc = H.oracle_scores(prob, 0)
    idx, c = H.oracle_select(prob, sc, wl.k)
    o_ref, l_ref = H.oracle_attention(prob, 0, idx, c)
    H.check_outputs(step.o[0], o_ref, step.lse[0], l_ref, torch.bfloat16, what="padding")


# ---------------------------------------------------------------------------
# Full-size workloads, drawn with the benchmark's seeds (its first input
# replica) and launched through the same prepared call list, so every kernel
# runs in the launch configuration the benchmark times.  Decode: scores and
# selections of every row against the oracle; outputs end to end on sampled
# rows whose oracle index sets the GPU reproduced.  Prefill: sampled rows.
# ---------------------------------------------------------------------------


def _row_subset(prob, rows):
    import dataclasses

    r = torch.as_tensor(rows, dtype=torch.long, device=prob.seq_of_row.device)
    return dataclasses.replace(prob, seq_of_row=prob.seq_of_row[r], pos_of_row=prob.pos_of_row[r],
                               idx_q=[x[r] for x in prob.idx_q], idx_w=[x[r] for x in prob.idx_w],
                               q=[x[:, r] for x in prob.q])


def _same_rows(gi, gc, oi, oc):
    gi, gc = np.asarray(gi), np.asarray(gc)
    return [r for r in range(len(oc))
            if gc[r] == oc[r] and np.array_equal(gi[r, :gc[r]], oi[r, :oc[r]])]


def _spread(rows, n=16):
    if len(rows) <= n:
        return list(rows)
    return [rows[int(round(i * (len(rows) - 1) / (n - 1)))] for i in range(n)]


@pytest.mark.parametrize("integer", [True, False])
@pytest.mark.parametrize("name", ["hysparse2", "csa", "csa2"])
def test_full_size_decode(name, integer, dev):
    from index_reuse_amd.pipeline import Step

    wl = synth.WORKLOADS[name]
    _flush("case full-size %s integer=%s" % (name, integer))
    prob = synth.make_problem(wl, device=dev, integer=integer)
    step = Step(prob)
    stream = torch.cuda.current_stream().cuda_stream
    for _, c in step.prepare():
        c(stream)
    torch.cuda.synchronize()
    cpu = H.move(prob, "cpu")
    R = cpu.n_rows

    sc = H.oracle_scores(cpu, 0)
    g = step.scores[0].cpu().double().numpy()
    valid = ~np.isnan(sc)
    tau = None if integer else H.fp32_score_bound(cpu, 0)
    if integer:
        assert np.array_equal(g[valid], sc[valid])
    else:
        err = np.abs(g - np.nan_to_num(sc))
        assert np.all(err[valid] <= np.broadcast_to(tau[:, None], sc.shape)[valid])
    gi = [t.cpu().numpy() for t in step.idx]
    gc = [t.cpu().numpy() for t in step.count]
    if wl.block:
        idx, cnt, pool, pc = H.oracle_select(cpu, sc, wl.k, block=wl.block,
                                             max_blocks=wl.max_blocks)
        H.check_indices(gi[0], gc[0], idx, cnt, sc, tau, win_lo=H.win_lo(cpu))
        gpool, gpc = step.pool.cpu().numpy(), step.pool_count.cpu().numpy()
        pool_same = [r for r in range(R) if gpc[r] == pc[r] and np.array_equal(gpool[r], pool[r])]
        if integer:
            assert len(pool_same) == R
        assert pool_same, "no row reproduced the oracle's block pool"
        rs = H.oracle_scores(cpu, 1, cand=pool, cand_count=pc)
        gr = step.scores[1].cpu().double().numpy()
        tau1 = None if integer else H.fp32_score_bound(cpu, 1)
        for r in pool_same:
            v = ~np.isnan(rs[r])
            if integer:
                assert np.array_equal(gr[r, v], rs[r, v])
            else:
                assert np.all(np.abs(gr[r, v] - rs[r, v]) <= tau1[r])
        ridx, rcnt = H.oracle_select(cpu, rs, wl.k, cand=pool, cand_count=pc)
        H.check_indices(gi[1], gc[1], ridx, rcnt, rs, tau1, rows=pool_same, positions=pool,
                        win_lo=H.win_lo(cpu))
        oidx, ocnt = [idx, ridx], [cnt, rcnt]
        same = [sorted(set(_same_rows(gi[0], gc[0], idx, cnt))),
                sorted(set(_same_rows(gi[1], gc[1], ridx, rcnt)) & set(pool_same))]
    else:
        idx, cnt = H.oracle_select(cpu, sc, wl.k)
        H.check_indices(gi[0], gc[0], idx, cnt, sc, tau, win_lo=H.win_lo(cpu))
        oidx, ocnt = [idx], [cnt]
        same = [_same_rows(gi[0], gc[0], idx, cnt)]
    for c in range(len(cpu.q)):
        if integer:
            assert len(same[c]) == R
        assert same[c], "call %d: no row reproduced the oracle's index set" % c
        rows = _spread(same[c])
        o_ref, l_ref = H.oracle_attention(cpu, c, oidx[c], ocnt[c], rows=rows)
        H.check_outputs(step.o[c][:, rows], o_ref, step.lse[c][:, rows], l_ref, wl.attn_dtype,
                        what="%s call %d rows %s" % (name, c, rows))


def _dsa_full_rows():
    """128 sampled rows of the 64K prefill: the first and last row of every
    8192-row block, both sides of the budget edge (t + 1 = 2048), and rows
    drawn uniformly from the rest (fixed seed)."""
    rows = set()
    for b in range(8):
        rows |= {8192 * b, 8192 * b + 8191}
    rows |= {1, 2, 2046, 2047, 2048, 2049, 30001, 49152}
    rng = np.random.default_rng(2026)
    while len(rows) < 128:
        rows.add(int(rng.integers(0, 65536)))
    return sorted(rows)


DSA_FULL_ROWS = _dsa_full_rows()


@pytest.mark.parametrize("integer", [True, False])
def test_full_size_prefill(integer, dev):
    """DSA prefill over the whole 64K-token sequence in the benchmark's row
    blocks; sampled rows (both sides of the budget edge, of a block edge, and
    the last row) against the oracle."""
    from index_reuse_amd.pipeline import PrefillStep

    wl = synth.DSA
    _flush("case full-size dsa integer=%s" % integer)
    prob = synth.make_problem(wl, device=dev, integer=integer)
    step = PrefillStep(prob, row_block=8192)
    step.run()
    torch.cuda.synchronize()
    rows = DSA_FULL_ROWS
    sub = H.move(_row_subset(prob, rows), "cpu")
    del prob
    sc = H.oracle_scores(sub, 0)
    tau = None if integer else H.fp32_score_bound(sub, 0)
    idx, cnt = H.oracle_select(sub, sc, wl.k)
    assert list(cnt) == [min(wl.k, t + 1) for t in rows]
    assert max(rows) < step.idx.shape[0] == step.count.shape[0] == step.R
    gi = step.idx.cpu().numpy()[rows]
    gc = step.count.cpu().numpy()[rows]
    H.check_indices(gi, gc, idx, cnt, sc, tau, win_lo=H.win_lo(sub))
    same = _same_rows(gi, gc, idx, cnt)
    if integer:
        assert len(same) == len(rows)
    assert same
    o_ref, l_ref = H.oracle_attention(sub, 0, idx, cnt, rows=same)
    # PrefillStep keeps one [n_sets, R, hq, dv] output (and [n_sets, R, hq]
    # LSE) for all rows: pick the sampled rows on dimension 1.
    pick = [rows[i] for i in same]
    assert step.o.dim() == 4 and step.lse.dim() == 3
    assert max(pick) < step.o.shape[1] == step.lse.shape[1] == step.R
    sel = torch.tensor(pick, dtype=torch.long, device=step.o.device)
    H.check_outputs(step.o.index_select(1, sel), o_ref, step.lse.index_select(1, sel), l_ref,
                    wl.attn_dtype, what="dsa rows %s" % pick)


@pytest.mark.parametrize("hkv", [1, 2])
def test_attention_many_splits_single_row(hkv, dev):
    """One decode row with window + top-k far above one workgroup's 2048
    entries and few KV heads: the planner wants more than 64 entry splits,
    and must stop at the 64 the split merge handles."""
    wl = synth.HYSPARSE2.replace(n_seqs=1, seq_lens_override=(9000,), k=4096, hq=8 * hkv,
                                 hkv=hkv, n_qsets=1)
    prob = synth.make_problem(wl, device="cpu")
    _flush("case many splits hkv=%d" % hkv)
    p, step = _step(prob, dev)
    sc = H.oracle_scores(prob, 0)
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    assert cnt[0] == 4096
    step.run_attention(idx=[torch.from_numpy(idx).to(dev)], count=[torch.from_numpy(cnt).to(dev)])
    torch.cuda.synchronize()
    o_ref, l_ref = H.oracle_attention(prob, 0, idx, cnt)
    H.check_outputs(step.o[0], o_ref, step.lse[0], l_ref, torch.bfloat16, what="splits")


def test_reindex_leaves_caches_unchanged(dev):
    """A Reindex layer only rescores and reselects: after a whole CSA2 layer
    group (Full, Reindex, Reuse) the index-key cache and the main KV are
    bitwise what they were ("CSA, HCA and CSA2", section 5.1: Reindex writes
    no KV)."""
    wl, _ = CASES["csa2"]
    p, step = _step(synth.make_problem(wl, device="cpu"), dev)
    before = [p.kidx.pool.clone(), p.k.pool.clone(), p.k.scale.clone()]
    step.run()
    torch.cuda.synchronize()
    for a, b in zip(before, [p.kidx.pool, p.k.pool, p.k.scale]):
        assert torch.equal(a, b)


def test_select_workspace_shared_across_row_counts(dev):
    """Chunk-path selections (rows longer than 65536 elements) of different
    row counts share one workspace, in alternation: every result stays
    bit-exact (nothing a call leaves in the workspace reaches the next)."""
    from index_reuse_amd import Rows
    from index_reuse_amd.binding import prepare_topk_select

    import oracle

    calls = []
    for R, S, seed in ((5, 70000, 301), (3, 100000, 302), (2, 80000, 303)):
        scores = synth.small_ints((R, S), seed=seed, lo=-30, hi=30)
        scores[scores == 0] = -0.0
        so = torch.zeros(R, dtype=torch.int32)
        po = torch.tensor([S - 1 - 11 * r for r in range(R)], dtype=torch.int32)
        sl = torch.tensor([S], dtype=torch.int32)
        ref = oracle.topk_select(so, po, sl, 1, 16, scores.double().numpy(), 3000)
        rows = Rows(so.to(dev), po.to(dev), sl.to(dev), 1, 16)
        idx = torch.empty(R, 3000, dtype=torch.int32, device=dev)
        cnt = torch.empty(R, dtype=torch.int32, device=dev)
        calls.append((rows, scores.to(dev), idx, cnt, ref))
    shared = None
    prepared = []
    for rows, sc, idx, cnt, ref in calls:
        pc = prepare_topk_select(rows, sc, 3000, idx, cnt)
        prepared.append(pc)
        if shared is None or pc.need > shared.numel():
            shared = torch.full((pc.need,), 0x5A, dtype=torch.uint8, device=dev)
    for pc in prepared:
        pc.ws, pc.ws_ptr = shared, shared.data_ptr()
    for rep in range(2):
        for pc, (rows, sc, idx, cnt, ref) in zip(prepared, calls):
            idx.fill_(7)
            pc()
            torch.cuda.synchronize()
            assert np.array_equal(cnt.cpu().numpy(), ref[1]), rep
            assert np.array_equal(idx.cpu().numpy(), ref[0]), rep


def test_check_indices_device(dev):
    """The device-side index check passes the oracle's selections and names
    the first bad row for planted mistakes (an index shifted into the window,
    a descending pair, a count above k, a padding slot, a padding row that
    leaked a count)."""
    from index_reuse_amd import SAError, check_indices

    wl, integer, prob = _problem("hysparse2_int")
    p, step = _step(prob, dev)
    sc = H.oracle_scores(prob, 0)
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    rows = step.rows
    check_indices(rows, torch.from_numpy(idx).to(dev), torch.from_numpy(cnt).to(dev))
    wlo = H.win_lo(prob)
    r0 = int(np.argmax(cnt))
    cases = []
    a = idx.copy()
    a[r0, cnt[r0] - 1] = wlo[r0]
    cases.append((a, cnt, r0, "outside"))
    a = idx.copy()
    a[r0, 0], a[r0, 1] = a[r0, 1], a[r0, 0]
    cases.append((a, cnt, r0, "ascending"))
    c = cnt.copy()
    c[r0] = wl.k + 1
    cases.append((idx, c, r0, "count"))
    r1 = int(np.argmin(cnt))
    a = idx.copy()
    a[r1, wl.k - 1] = 3
    cases.append((a, cnt, r1, "padding slot" if cnt[r1] < wl.k else "ascending"))
    for bad_idx, bad_cnt, row, what in cases:
        with pytest.raises(SAError, match="row %d: .*%s" % (row, what)):
            check_indices(rows, torch.from_numpy(np.ascontiguousarray(bad_idx)).to(dev),
                          torch.from_numpy(np.ascontiguousarray(bad_cnt)).to(dev))


def test_peak_probes_run(dev):
    """The achievable-peak probes run and report plausible MI355X rates (a
    streaming read between 1 and 8 TB/s; dense MFMA loops above 100 TFLOP/s
    and below the 2.5 / 5.0 PF dense peaks)."""
    from index_reuse_amd import binding as B

    _flush("case peak probes")
    gbs = B.peak_read_gbs(1 << 30)
    bf16 = B.peak_mfma_tflops("bf16", iters=512)
    fp8 = B.peak_mfma_tflops("fp8", iters=256)
    assert 1000 < gbs < 8000, gbs
    assert 100 < bf16 < 2500 * 1.02, bf16
    assert 100 < fp8 < 5000 * 1.02, fp8
