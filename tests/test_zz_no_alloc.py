"""The allocation-free attention entry point, through the C ABI: it must give
exactly what sparse_attn_gather_fwd gives (same kernels, the split partials in
a static per-device array instead of the caller's workspace), on two calls in
a row with the second smaller than the first, and reject a call whose
partials exceed the static array."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import index_reuse_amd

    return index_reuse_amd.load()


def _call_pair(lib, wl, seed):
    from index_reuse_amd import binding as B
    from index_reuse_amd.pipeline import Step

    prob = synth.make_problem(wl, device="cpu", seed_base=seed)
    p = H.move(prob, "cuda")
    step = Step(p)
    sc = H.oracle_scores(prob, 0)
    idx, cnt = H.oracle_select(prob, sc, wl.k)
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    q = p.q[0]
    outs = []
    for noalloc in (False, True):
        o = torch.full((q.shape[0], q.shape[1], wl.hq, wl.dv), float("nan"), dtype=q.dtype,
                       device="cuda")
        lse = torch.full((q.shape[0], q.shape[1], wl.hq), float("nan"), dtype=torch.float32,
                         device="cuda")
        d = B.attn_desc(step.rows, q, step.k, step.v, ti, tc, o, lse, step.scale, wl.dv)
        stream = torch.cuda.current_stream().cuda_stream
        if noalloc:
            st = lib.sparse_attn_gather_fwd_noalloc(ctypes.byref(d), stream)
        else:
            need = int(lib.sa_workspace_size(B.SA_OP_ATTN_GATHER_FWD, ctypes.byref(d)))
            assert need > 0, "the case must use split partials"
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            st = lib.sparse_attn_gather_fwd(ctypes.byref(d), ws.data_ptr(), need, stream)
        assert st == 0, lib.sa_last_error()
        torch.cuda.synchronize()
        outs.append((o, lse))
    (o0, l0), (o1, l1) = outs
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    o_ref, l_ref = H.oracle_attention(prob, 0, idx, cnt)
    H.check_outputs(o1, o_ref, l1, l_ref, wl.attn_dtype, what="noalloc")
    return int(lib.sa_workspace_size(B.SA_OP_ATTN_GATHER_FWD, ctypes.byref(d)))


def test_noalloc_matches_workspace_entry_point(lib):
    big = synth.CSA.replace(n_seqs=8, seq_len=16384, tail_variant=True)
    small = synth.CSA.replace(n_seqs=2, seq_len=4096, tail_variant=True)
    n_big = _call_pair(lib, big, 901)
    n_small = _call_pair(lib, small, 902)
    print("partials: %d then %d bytes" % (n_big, n_small), flush=True)
    assert n_small < n_big


def test_noalloc_rejects_oversized_call(lib):
    """More split partials than the static array holds (40 query sets of 64
    heads over 512-wide rows with an 8192-entry window, which needs at least
    four entry splits): SA_ERR_WORKSPACE and no launch (the output keeps its
    contents)."""
    from index_reuse_amd import binding as B
    from index_reuse_amd.pipeline import Step

    wl = synth.CSA.replace(n_seqs=4, seq_len=40000, n_qsets=40, window=8192)
    prob = synth.make_problem(wl, device="cpu")
    p = H.move(prob, "cuda")
    step = Step(p)
    idx = torch.full((4, wl.k), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(4, dtype=torch.int32, device="cuda")
    o = torch.full((40, 4, 64, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    d = B.attn_desc(step.rows, p.q[0], step.k, None, idx, cnt, o, None, step.scale, 512)
    need = int(lib.sa_workspace_size(B.SA_OP_ATTN_GATHER_FWD, ctypes.byref(d)))
    assert need > 64 << 20, need
    st = lib.sparse_attn_gather_fwd_noalloc(ctypes.byref(d), torch.cuda.current_stream().cuda_stream)
    assert st == -5 and b"static scratch" in lib.sa_last_error()
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)
