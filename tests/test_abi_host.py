"""Host-only checks of the C ABI (no GPU): the library loads, exports every
symbol the header declares, and rejects malformed descriptors before any
device work."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (binds the HIP runtime before the library)

import index_reuse_amd as ira
from index_reuse_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ira.LIB_PATH):
        import index_reuse_amd.build as bld

        bld.build()
    return ira.load()


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, re.M))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared == set(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_exports_peak_probes(lib):
    """include/sa_peak.h (measurement probes) is exported by the same library."""
    declared = _declared_functions(os.path.join(ROOT, "include", "sa_peak.h"))
    assert declared == set(B.PEAK_EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_peak_probes_reject_bad_arguments(lib):
    """Invalid probe arguments are rejected on the host (no launch)."""
    assert lib.sa_peak_mfma(3, 1, None, 1, None) < 0
    assert lib.sa_peak_read(None, 16, None, 1, None) < 0


def test_abi_version(lib):
    v = ira.abi_version()
    assert v >> 16 == 3 and v & 0xFFFF == 1


def test_struct_layout_matches_c_compiler(tmp_path):
    """Every ctypes descriptor has the size and field offsets gcc gives the
    header's structs."""
    import subprocess

    structs = [B.sa_cache, B.sa_rows, B.sa_index_desc, B.sa_topk_desc, B.sa_attn_desc]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "sparse_attn.h"',
             "int main(void) {"]
    for st in structs:
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (st.__name__, st.__name__))
        for f, _ in st._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));'
                         % (st.__name__, f, st.__name__, f))
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I" + os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = dict(l.split() for l in subprocess.check_output([str(exe)]).decode().splitlines())
    for st in structs:
        assert int(got[st.__name__]) == ctypes.sizeof(st), st.__name__
        for f, _ in st._fields_:
            assert int(got[st.__name__ + "." + f]) == getattr(st, f).offset, (st.__name__, f)


def _rows(n=4):
    return B.sa_rows(n, 1, 0x1000, 0x2000, 0x3000, 1, 0)


def _status(fn, desc):
    return fn(ctypes.byref(desc), None, 0, None)


def test_index_score_validation(lib):
    k = B.sa_cache(0x10000, None, None, 64, 8, 1, 64, 128, 0, B.SA_BF16, 0)
    d = B.sa_index_desc(_rows(), 0x20000, 0x30000, k, 16, 64, None, None, 0, 0, 0x40000, 4096,
                        None, 0, 0)
    bad = B.sa_index_desc.from_buffer_copy(d)
    bad.scores = None
    assert _status(lib.sparse_index_score, bad) == -1
    bad = B.sa_index_desc.from_buffer_copy(d)
    bad.dim = 96
    assert _status(lib.sparse_index_score, bad) == -4
    assert b"dim 64 or 128" in lib.sa_last_error()
    bad = B.sa_index_desc.from_buffer_copy(d)
    bad.k.width = 32
    assert _status(lib.sparse_index_score, bad) == -2
    bad = B.sa_index_desc.from_buffer_copy(d)
    bad.k.dtype = B.SA_FP4_E2M1
    assert _status(lib.sparse_index_score, bad) == -3
    bad = B.sa_index_desc.from_buffer_copy(d)
    bad.k.row_stride = 100  # below 128 bytes and not 16-aligned
    assert _status(lib.sparse_index_score, bad) == -2
    bad = B.sa_index_desc.from_buffer_copy(d)
    bad.rows.stride = 0
    assert _status(lib.sparse_index_score, bad) == -2
    assert lib.sa_workspace_size(B.SA_OP_INDEX_SCORE, ctypes.byref(d)) == 0


def test_index_score_fused_selection_validation(lib):
    """The fused selection: scores may be NULL, the workspace holds one pass
    of rows' scores plus the selection's workspace, and the selection's
    descriptor is validated like sparse_topk_select's."""
    k = B.sa_cache(0x10000, None, None, 64, 8, 1, 64, 128, 0, B.SA_BF16, 0)
    d = B.sa_index_desc(_rows(), 0x20000, 0x30000, k, 16, 64, None, None, 0, 0, None, 4096,
                        None, 0, 0)
    assert _status(lib.sparse_index_score, d) == -1  # neither scores nor sel
    sel = B.sa_topk_desc(_rows(), None, 0, None, None, 0, 8, 0x50000, 0x60000, 8, 0, 0, 0, None,
                         None)
    d.sel = ctypes.addressof(sel)
    size = lambda: lib.sa_workspace_size(B.SA_OP_INDEX_SCORE, ctypes.byref(d))
    whole = size()
    assert whole >= 4 * 4096 * 4 and whole != ctypes.c_size_t(-1).value
    d.row_block = 2
    half = size()
    assert 2 * 4096 * 4 <= half < whole
    assert _status(lib.sparse_index_score, d) == -5  # no workspace given
    d.row_block = -1
    assert _status(lib.sparse_index_score, d) == -2
    d.row_block = 0
    d.reserved = 1
    assert _status(lib.sparse_index_score, d) == -2
    d.reserved = 0
    sel.idx_stride = 4  # below k
    assert size() == ctypes.c_size_t(-1).value
    assert b"idx_stride < k" in lib.sa_last_error()


def test_topk_validation(lib):
    d = B.sa_topk_desc(_rows(), 0x1000, 64, None, None, 0, 8, 0x2000, 0x3000, 4, 0, 0, 0, None,
                       None)
    assert _status(lib.sparse_topk_select, d) == -2  # idx_stride < k
    d.idx_stride = 8
    d.k = 0
    assert _status(lib.sparse_topk_select, d) == -2  # nothing to do
    d.k = 8
    d.pool = 0x4000
    d.pool_count = 0x5000
    d.block, d.max_blocks, d.pool_stride = 8, 4, 16
    assert _status(lib.sparse_topk_select, d) == -2  # pool_stride < max_blocks*block
    d.cand, d.cand_count, d.cand_stride, d.pool_stride = 0x6000, 0x7000, 32, 32
    assert _status(lib.sparse_topk_select, d) == -4  # pool needs full-domain scores


def test_attn_validation_and_workspace(lib):
    k = B.sa_cache(0x10000, None, 0x100, 64, 512, 8, 128, 2048, 0, B.SA_BF16, 0)
    v = B.sa_cache(0x20000, None, 0x100, 64, 512, 8, 128, 2048, 0, B.SA_BF16, 0)
    rows = B.sa_rows(32, 32, 0x1000, 0x2000, 0x3000, 1, 128)
    d = B.sa_attn_desc(rows, 6, 64, 0x40000, B.SA_BF16, 128, k, v, 0, 1024, 0x5000, 0x6000,
                       0.088, B.SA_BF16, 0x70000, None)
    ws = lib.sa_workspace_size(B.SA_OP_ATTN_GATHER_FWD, ctypes.byref(d))
    assert ws != ctypes.c_size_t(-1).value
    assert ws % 4 == 0
    assert _status(lib.sparse_attn_gather_fwd, d) == -5 if ws else True  # no workspace given
    bad = B.sa_attn_desc.from_buffer_copy(d)
    bad.n_heads_q = 60
    assert _status(lib.sparse_attn_gather_fwd, bad) == -2
    bad = B.sa_attn_desc.from_buffer_copy(d)
    bad.q_dtype = B.SA_F32
    assert _status(lib.sparse_attn_gather_fwd, bad) == -3
    bad = B.sa_attn_desc.from_buffer_copy(d)
    bad.v.block_table = 0x200
    assert _status(lib.sparse_attn_gather_fwd, bad) == -2
    bad = B.sa_attn_desc.from_buffer_copy(d)
    bad.k.width = bad.v.width = bad.d_v = 96
    assert _status(lib.sparse_attn_gather_fwd, bad) == -4
    bad = B.sa_attn_desc.from_buffer_copy(d)
    bad.k.dtype = B.SA_FP4_E2M1
    assert _status(lib.sparse_attn_gather_fwd, bad) == -4  # FP4 needs v_from_k
    bad = B.sa_attn_desc.from_buffer_copy(d)
    bad.rows.window = 131072 - 1024 + 1  # window + idx_stride beyond the per-row limit
    assert _status(lib.sparse_attn_gather_fwd, bad) == -4
    bad = B.sa_attn_desc.from_buffer_copy(d)
    bad.k.row_stride = bad.v.row_stride = 1 << 31  # strides must stay below 2^31
    assert _status(lib.sparse_attn_gather_fwd, bad) == -2


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(B.SAError):
        saved = B._lib
        B._lib = None
        try:
            B.load(str(tmp_path / "missing.so"))
        finally:
            B._lib = saved
