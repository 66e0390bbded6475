"""Pins of the benchmark's work models against the figures the pages print
(no GPU).

  * "CSA, HCA and CSA2", section 3.1 (the cost breakdown of one layer group)
    and section 6.2 (the 1M-context state count): one Full, two Reindex and
    five Reuse layers score 8 x 32768 = 262144 entries per query flat, but
    32768 + 2 x 4096 = 40960 hierarchically with a 4096-entry pool; at
    262144 entries with a 16384-entry pool, 2,097,152 against 294,912.  The
    CSA2 decode workload's own group (1 Full, 1 Reindex, 3 Reuse) gives
    278,528 against 1,310,720.  The pool sizes are taken from the oracle's
    block-max pool (512 or 2048 blocks of 8), not assumed.
  * "Lecture 10 - Hybrid LLMs", section 5.3 and exercise 7: the 64K DSA
    prefill's sparse main attention of about 0.66 PFLOP over 61 layers at
    81,920 operations per selected (query, key) pair is 132,121,600 selected
    pairs per layer = sum_t min(2048, t + 1); the indexer's 2.15 PFLOP is
    2,147,516,416 causal pairs x 16,384 operations x 61 layers.
"""
import types

import numpy as np
import pytest

import bench
import synth


@pytest.mark.parametrize("n,pool,plan,want", [
    (32768, 4096, (1, 2, 5), (262144, 40960)),
    (262144, 16384, (1, 2, 5), (2097152, 294912)),
    (262144, 16384, (1, 1, 3), (1310720, 278528)),
])
def test_layer_group_counts_closed_form(n, pool, plan, want):
    assert bench.layer_group_index_work(n, pool, *plan) == want


@pytest.mark.parametrize("n,max_blocks,plan,want", [
    (32768, 512, (1, 2, 5), (262144, 40960)),
    (262144, 2048, (1, 2, 5), (2097152, 294912)),
    (262144, 2048, (1, 1, 3), (1310720, 278528)),
])
def test_layer_group_counts_from_oracle_pool(orc, n, max_blocks, plan, want):
    """The pool a Full layer builds over n entries with max_blocks blocks of 8
    (the oracle's block-max pool on arbitrary scores) has 8 x max_blocks
    members; fed to the work model it reproduces the pages' counts."""
    rng = np.random.default_rng(n + max_blocks)
    scores = rng.standard_normal((1, n))
    so, po, sl = np.zeros(1, np.int32), np.array([n - 1], np.int32), np.array([n], np.int32)
    _, _, pool, pc = orc.topk_select(so, po, sl, 1, 0, scores, 512, block=8,
                                     max_blocks=max_blocks)
    assert pc[0] == 8 * max_blocks
    members = pool[0, :pc[0]]
    assert np.all(np.diff(members) > 0) and members[0] >= 0 and members[-1] < n
    assert bench.layer_group_index_work(n, int(pc[0]), *plan) == want


def test_dsa_prefill_pairs():
    w = bench.prefill_work_rows(synth.DSA, np.arange(65536), 65536)
    assert w["pairs"] == 65536 * 65537 // 2 == 2_147_516_416
    assert w["attn_pairs"] == sum(min(2048, t + 1) for t in range(65536)) == 132_121_600
    # 0.66 PFLOP over 61 layers at 81,920 operations per pair (exercise 7)
    assert abs(w["attn_pairs"] * 81920 * 61 / 1e15 - 0.66) < 0.005
    # indexer: 64 heads x 128 channels x 2 per pair = 16,384; 2.15 PFLOP over 61 layers
    assert w["index_score"] == 2.0 * w["pairs"] * 64 * 128
    assert abs(w["index_score"] * 61 / 1e15 - 2.15) < 0.005
    # attention at this build's widths: 128 heads x (576 + 512) x 2 per pair
    assert w["attn_gather_fwd"] == 2.0 * 132_121_600 * 128 * (576 + 512)


def _fake_step(wl):
    import torch

    B = wl.n_seqs
    prob = types.SimpleNamespace(
        seq_of_row=torch.arange(B, dtype=torch.int32),
        pos_of_row=torch.tensor(wl.seq_lens(), dtype=torch.int32) - 1,
        seq_len=torch.tensor(wl.seq_lens(), dtype=torch.int32),
        q=[types.SimpleNamespace(shape=(wl.n_qsets,))])
    return types.SimpleNamespace(wl=wl, prob=prob, pool_count=None)


def test_hysparse2_decode_bytes():
    """The HySparse2 decode step's algorithmic bytes: the indexer reads every
    visible 64-wide bf16 key (32 x 32768 x 128 B) and writes its scores; the
    gather reads the window + top-k rows of K and V once for all 6 query sets
    (32 x 1152 x 8 heads x 256 B x 2), plus queries, outputs, LSE and
    indices."""
    st = _fake_step(synth.HYSPARSE2)
    n = 32 * 32768
    assert bench.algorithmic_bytes(st, "index_score") == n * 128 + 32 * 16 * (128 + 4) + n * 4
    kv = 32 * 1152 * 8 * 128 * 2 * 2
    qo = 6 * 32 * 64 * (128 + 128) * 2 + 6 * 32 * 64 * 4
    assert bench.algorithmic_bytes(st, "attn_gather_fwd") == kv + qo + 32 * 1024 * 4
    assert kv == 150_994_944


def test_dense_crossover():
    """Exercise 6 of "Lecture 10": with 1152-byte latent rows, 128-byte FP8
    index keys and k = 2048, sparse decode reads fewer bytes than dense once
    L > 2304; at L = 2048 it reads about 11% more (the page's table: 10%
    slower) and at 4096 dense reads 1.64x more."""
    assert bench.dense_crossover(1152, 128, 2048) == 2304
    sparse = lambda L: 128 * L + 1152 * 2048
    dense = lambda L: 1152 * L
    assert abs(sparse(2048) / dense(2048) - 1.111) < 0.001
    assert abs(dense(4096) / sparse(4096) - 1.64) < 0.005


def test_traffic_records_keyed_by_call(tmp_path, monkeypatch):
    """A counter record belongs to the call it names: the FA workload's
    dense attention call must not take the sparse attention call's record,
    and a record taken on other kernel sources is not used."""
    fam_hash = bench.source_hash("attn_gather_fwd")
    rec = "# test record\nsource_sha256: %s\ntraffic_bytes: 1234\n" % fam_hash
    (tmp_path / "attn_gather_fwd_hysparse2_traffic.txt").write_text(rec)
    (tmp_path / "index_score_hysparse2_traffic.txt").write_text(
        "source_sha256: 0000\ntraffic_bytes: 99\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.recorded_traffic("attn_gather_fwd", "hysparse2") == 1234.0
    assert bench.recorded_traffic("attn_gather_fwd_fa", "hysparse2") is None
    assert bench.recorded_traffic("index_score", "hysparse2") is None
    assert bench.recorded_traffic("attn_gather_fwd", "csa") is None
