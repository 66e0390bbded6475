"""ctypes binding of libsparse_attn.so.

Argument marshalling only: tensors become device pointers inside the C
descriptors of ``include/sparse_attn.h`` and every computation runs in the
library's HIP kernels.  torch provides device memory and the current stream.
There is no fallback: if the library is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_attn.so")

SA_F32, SA_BF16, SA_FP8_E4M3, SA_FP4_E2M1 = 0, 1, 2, 3
SA_OP_INDEX_SCORE, SA_OP_TOPK_SELECT, SA_OP_ATTN_GATHER_FWD = 0, 1, 2

_P = ctypes.c_void_p
_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float


class sa_cache(ctypes.Structure):
    _fields_ = [("data", _P), ("scale", _P), ("block_table", _P), ("page_size", _i32),
                ("max_pages", _i32), ("heads", _i32), ("width", _i32), ("row_stride", _i64),
                ("scale_stride", _i64), ("dtype", _i32), ("reserved", _i32)]


class sa_rows(ctypes.Structure):
    _fields_ = [("n_rows", _i32), ("n_seqs", _i32), ("seq_of_row", _P), ("pos_of_row", _P),
                ("seq_len", _P), ("stride", _i32), ("window", _i32)]


class sa_index_desc(ctypes.Structure):
    _fields_ = [("rows", sa_rows), ("q", _P), ("w", _P), ("k", sa_cache), ("n_heads", _i32),
                ("dim", _i32), ("cand", _P), ("cand_count", _P), ("cand_stride", _i32),
                ("skip_k", _i32), ("scores", _P), ("score_stride", _i64), ("sel", _P),
                ("row_block", _i32), ("reserved", _i32)]


class sa_topk_desc(ctypes.Structure):
    _fields_ = [("rows", sa_rows), ("scores", _P), ("score_stride", _i64), ("cand", _P),
                ("cand_count", _P), ("cand_stride", _i32), ("k", _i32), ("idx", _P),
                ("count", _P), ("idx_stride", _i32), ("block", _i32), ("max_blocks", _i32),
                ("pool_stride", _i32), ("pool", _P), ("pool_count", _P)]


class sa_attn_desc(ctypes.Structure):
    _fields_ = [("rows", sa_rows), ("n_qsets", _i32), ("n_heads_q", _i32), ("q", _P),
                ("q_dtype", _i32), ("d_v", _i32), ("k", sa_cache), ("v", sa_cache),
                ("v_from_k", _i32), ("idx_stride", _i32), ("idx", _P), ("count", _P),
                ("scale", _f32), ("o_dtype", _i32), ("o", _P), ("lse", _P), ("sink", _P),
                ("gate", _P)]


EXPORTS = ("sparse_index_score", "sparse_topk_select", "sparse_attn_gather_fwd",
           "sparse_attn_gather_fwd_noalloc", "sparse_attn_score", "sparse_check_indices",
           "sa_workspace_size", "sa_last_error", "sa_abi_version")
# include/sa_peak.h: achievable-peak probes (measurement only)
PEAK_EXPORTS = ("sa_peak_read", "sa_peak_mfma")

_lib = None


class SAError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Load the HIP library (after torch, so that it binds to the HIP runtime
    torch already mapped).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise SAError("libsparse_attn.so not built: run `python -m index_reuse_amd.build` "
                      "(or __graft_entry__.build())")
    L = ctypes.CDLL(path)
    for name in ("sparse_index_score", "sparse_topk_select", "sparse_attn_gather_fwd"):
        getattr(L, name).restype = _i32
    L.sparse_index_score.argtypes = [ctypes.POINTER(sa_index_desc), _P, ctypes.c_size_t, _P]
    L.sparse_topk_select.argtypes = [ctypes.POINTER(sa_topk_desc), _P, ctypes.c_size_t, _P]
    L.sparse_attn_gather_fwd.argtypes = [ctypes.POINTER(sa_attn_desc), _P, ctypes.c_size_t, _P]
    L.sparse_attn_gather_fwd_noalloc.restype = _i32
    L.sparse_attn_gather_fwd_noalloc.argtypes = [ctypes.POINTER(sa_attn_desc), _P]
    L.sparse_attn_score.restype = _i32
    L.sparse_attn_score.argtypes = [ctypes.POINTER(sa_attn_desc), _P, _i64, _P]
    L.sparse_check_indices.restype = _i32
    L.sparse_check_indices.argtypes = [ctypes.POINTER(sa_topk_desc), _P, _P]
    L.sa_workspace_size.restype = ctypes.c_size_t
    L.sa_workspace_size.argtypes = [_i32, _P]
    L.sa_last_error.restype = ctypes.c_char_p
    L.sa_abi_version.restype = _i32
    L.sa_peak_read.restype = _i32
    L.sa_peak_read.argtypes = [_P, ctypes.c_size_t, _P, _i32, _P]
    L.sa_peak_mfma.restype = _i32
    L.sa_peak_mfma.argtypes = [_i32, _i32, _P, _i32, _P]
    _lib = L
    return L


def abi_version() -> int:
    return int(load().sa_abi_version())


def _check(status: int):
    if status != 0:
        msg = load().sa_last_error().decode(errors="replace")
        raise SAError("status %d: %s" % (status, msg))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return SA_FP8_E4M3
    raise SAError("unsupported dtype %s" % t.dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dense(t: Optional[torch.Tensor], name: str, rows: bool = False):
    """The descriptors pass a base pointer (plus a row stride for ``rows``
    tensors): the tensor must be contiguous (``rows``: each row contiguous)."""
    if t is None:
        return
    ok = t.stride(-1) == 1 if rows and t.dim() >= 1 else t.is_contiguous()
    if rows and t.dim() > 2:
        ok = ok and t[0].is_contiguous()
    if not ok:
        raise SAError("%s must be %s" % (name, "row-contiguous" if rows else "contiguous"))


# ---------------------------------------------------------------------------
# Python-side views of the descriptor parts
# ---------------------------------------------------------------------------


@dataclass
class Rows:
    seq_of_row: torch.Tensor  # int32 [R]
    pos_of_row: torch.Tensor  # int32 [R]
    seq_len: torch.Tensor     # int32 [B]
    stride: int = 1
    window: int = 0

    def c(self) -> sa_rows:
        return sa_rows(int(self.seq_of_row.numel()), int(self.seq_len.numel()),
                       _ptr(self.seq_of_row), _ptr(self.pos_of_row), _ptr(self.seq_len),
                       int(self.stride), int(self.window))


@dataclass
class Cache:
    """A paged cache: ``pool`` is [n_pages, page_size, heads, width] (or
    [n_seqs, cap, heads, width] with ``block_table=None``); FP4 pools hold
    bytes [.., width/2] with ``scale`` [.., width/16]."""

    pool: torch.Tensor
    block_table: Optional[torch.Tensor]
    heads: int
    width: int
    fp4: bool = False
    scale: Optional[torch.Tensor] = None

    def c(self) -> sa_cache:
        p = self.pool
        page_size = int(p.shape[1])
        if self.block_table is not None:
            max_pages = int(self.block_table.shape[1])
        else:
            max_pages = 1
        row_stride = p.stride(1) * p.element_size()
        dtype = SA_FP4_E2M1 if self.fp4 else _dt(p)
        scale_stride = 0
        if self.fp4:
            scale_stride = self.scale.stride(1) * self.scale.element_size()
        return sa_cache(_ptr(p), _ptr(self.scale), _ptr(self.block_table), page_size, max_pages,
                        int(self.heads), int(self.width), row_stride, scale_stride, dtype, 0)


def _cache_struct(c: Cache) -> sa_cache:
    return c.c()


_ws_cache = {}


def workspace(nbytes: int, device, op: int) -> Optional[torch.Tensor]:
    """A cached device workspace of at least ``nbytes`` bytes for entry point
    ``op`` (no entry point reads what an earlier call left in it; calls on
    the current stream run one after another, so they can share it)."""
    if nbytes == 0:
        return None
    key = (torch.device(device).index, op)
    t = _ws_cache.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = t
    return t


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------


def index_desc(rows: Rows, q, w, k: Cache, scores, cand=None, cand_count=None,
               skip_k: int = 0, sel: Optional["sa_topk_desc"] = None, row_block: int = 0,
               n_slots: Optional[int] = None) -> sa_index_desc:
    """``sel`` (a topk descriptor, kept alive by the caller) asks for the
    fused selection; ``scores`` may then be None with ``n_slots`` giving the
    score capacity per row."""
    _dense(q, "q")
    _dense(w, "w")
    _dense(scores, "scores", rows=True)
    _dense(cand, "cand", rows=True)
    _dense(cand_count, "cand_count")
    stride = int(scores.stride(0)) if scores is not None else int(n_slots)
    sel_ptr = None if sel is None else ctypes.addressof(sel)
    return sa_index_desc(rows.c(), _ptr(q), _ptr(w), k.c(), int(q.shape[1]), int(q.shape[2]),
                         _ptr(cand), _ptr(cand_count), 0 if cand is None else int(cand.stride(0)),
                         int(skip_k), _ptr(scores), stride, sel_ptr, int(row_block), 0)


def index_score(rows: Rows, q: torch.Tensor, w: torch.Tensor, k: Cache,
                scores: Optional[torch.Tensor] = None, n_slots: Optional[int] = None,
                cand: Optional[torch.Tensor] = None, cand_count: Optional[torch.Tensor] = None,
                skip_k: int = 0):
    """Indexer scores [R, S] float32 (see sparse_index_score; ``skip_k``: the
    dense route)."""
    L = load()
    if scores is None:
        S = int(cand.shape[1]) if cand is not None else int(n_slots)
        scores = torch.empty(int(q.shape[0]), S, dtype=torch.float32, device=q.device)
    d = index_desc(rows, q, w, k, scores, cand, cand_count, skip_k)
    _check(L.sparse_index_score(ctypes.byref(d), None, 0, _stream()))
    return scores


def topk_desc(rows: Rows, scores, k: int, idx, count, cand=None, cand_count=None, block=0,
              max_blocks=0, pool=None, pool_count=None) -> sa_topk_desc:
    """``scores`` may be None for the ``sel`` of a fused index call."""
    _dense(scores, "scores", rows=True)
    for t, n in ((idx, "idx"), (cand, "cand"), (pool, "pool")):
        _dense(t, n, rows=True)
    for t, n in ((count, "count"), (cand_count, "cand_count"), (pool_count, "pool_count")):
        _dense(t, n)
    return sa_topk_desc(rows.c(), _ptr(scores), 0 if scores is None else int(scores.stride(0)),
                        _ptr(cand), _ptr(cand_count),
                        0 if cand is None else int(cand.stride(0)), int(k), _ptr(idx), _ptr(count),
                        0 if idx is None else int(idx.stride(0)), int(block), int(max_blocks),
                        0 if pool is None else int(pool.stride(0)), _ptr(pool), _ptr(pool_count))


def topk_select(rows: Rows, scores: torch.Tensor, k: int, cand=None, cand_count=None,
                block: int = 0, max_blocks: int = 0, idx=None, count=None, pool=None,
                pool_count=None):
    """Window + top-k (and optionally the block-max pool).  Returns
    (idx, count) or (idx, count, pool, pool_count)."""
    L = load()
    R, dev = int(scores.shape[0]), scores.device
    if k > 0 and idx is None:
        idx = torch.empty(R, k, dtype=torch.int32, device=dev)
        count = torch.empty(R, dtype=torch.int32, device=dev)
    if block > 0 and pool is None:
        pool = torch.empty(R, max_blocks * block, dtype=torch.int32, device=dev)
        pool_count = torch.empty(R, dtype=torch.int32, device=dev)
    d = topk_desc(rows, scores, k, idx, count, cand, cand_count, block, max_blocks, pool,
                  pool_count)
    need = int(L.sa_workspace_size(SA_OP_TOPK_SELECT, ctypes.byref(d)))
    if need == ctypes.c_size_t(-1).value:
        _check(-2)
    ws = workspace(need, scores.device, SA_OP_TOPK_SELECT)
    _check(L.sparse_topk_select(ctypes.byref(d), _ptr(ws), need, _stream()))
    if block > 0:
        return idx, count, pool, pool_count
    return idx, count


CHECK_CODES = {1: "count out of range", 2: "index outside the row's candidates",
               3: "indices not strictly ascending", 4: "padding slot not -1"}


def check_indices(rows: Rows, idx: torch.Tensor, count: torch.Tensor, k: Optional[int] = None,
                  candidate_mode: bool = False):
    """Check an index tensor on the device (sparse_check_indices) and raise
    SAError naming the first failing row; synchronises the stream."""
    L = load()
    k = int(idx.shape[1]) if k is None else int(k)
    _dense(idx, "idx", rows=True)
    _dense(count, "count")
    cand = count if candidate_mode else None  # only its presence is read
    d = topk_desc(rows, idx, k, idx, count, cand=cand, cand_count=count)
    err = torch.empty(1, dtype=torch.int32, device=idx.device)
    _check(L.sparse_check_indices(ctypes.byref(d), _ptr(err), _stream()))
    word = int(err.item()) & 0xFFFFFFFF
    if word != 0xFFFFFFFF:
        raise SAError("index check failed at row %d: %s" % (word >> 3,
                                                           CHECK_CODES.get(word & 7, "?")))


def attn_desc(rows: Rows, q, k: Cache, v: Optional[Cache], idx, count, o, lse=None,
              scale: Optional[float] = None, d_v: Optional[int] = None, sink=None,
              gate=None) -> sa_attn_desc:
    n_qsets, R, hq, dqk = (int(x) for x in q.shape)
    if d_v is None:
        d_v = v.width if v is not None else k.width
    if scale is None:
        scale = dqk ** -0.5
    for t, n in ((q, "q"), (o, "o"), (lse, "lse"), (count, "count"), (sink, "sink"),
                 (gate, "gate")):
        _dense(t, n)
    _dense(idx, "idx", rows=True)
    if sink is not None and (sink.dtype != torch.float32 or sink.numel() != n_qsets * hq):
        raise SAError("sink must be float32 [n_qsets, n_heads_q]")
    if gate is not None and (gate.dtype != q.dtype or tuple(gate.shape) != (n_qsets, R, hq, d_v)):
        raise SAError("gate must be [n_qsets, R, n_heads_q, d_v] in the query dtype")
    vc = v.c() if v is not None else sa_cache()
    return sa_attn_desc(rows.c(), n_qsets, hq, _ptr(q), _dt(q), int(d_v), k.c(), vc,
                        1 if v is None else 0, 0 if idx is None else int(idx.stride(0)), _ptr(idx),
                        _ptr(count), float(scale), _dt(o), _ptr(o), _ptr(lse), _ptr(sink),
                        _ptr(gate))


def attn_gather_fwd(rows: Rows, q: torch.Tensor, k: Cache, v: Optional[Cache] = None,
                    idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                    scale: Optional[float] = None, d_v: Optional[int] = None,
                    o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    out_dtype=None, want_lse: bool = True, sink=None, gate=None):
    """Joint-softmax gather attention.  ``v=None`` means V is the first d_v
    channels of the K row; ``sink`` [n_qsets, hq] f32 and ``gate`` [n_qsets,
    R, hq, d_v] are the optional per-head sink bias and output sigmoid gate.
    Returns (o, lse)."""
    L = load()
    n_qsets, R, hq, dqk = (int(x) for x in q.shape)
    if d_v is None:
        d_v = v.width if v is not None else k.width
    if o is None:
        o = torch.empty(n_qsets, R, hq, d_v, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(n_qsets, R, hq, dtype=torch.float32, device=q.device)
    d = attn_desc(rows, q, k, v, idx, count, o, lse, scale, d_v, sink, gate)
    need = int(L.sa_workspace_size(SA_OP_ATTN_GATHER_FWD, ctypes.byref(d)))
    if need == ctypes.c_size_t(-1).value:
        _check(-2)
    ws = workspace(need, q.device, SA_OP_ATTN_GATHER_FWD)
    _check(L.sparse_attn_gather_fwd(ctypes.byref(d), _ptr(ws), need, _stream()))
    return o, lse


def score_desc(rows: Rows, q, k: Cache, lse, scale: Optional[float] = None) -> sa_attn_desc:
    """The attention descriptor fields sparse_attn_score reads."""
    n_qsets, R, hq, dqk = (int(x) for x in q.shape)
    if scale is None:
        scale = dqk ** -0.5
    _dense(q, "q")
    _dense(lse, "lse")
    return sa_attn_desc(rows.c(), n_qsets, hq, _ptr(q), _dt(q), dqk, k.c(), sa_cache(), 1, 0, None,
                        None, float(scale), _dt(q), None, _ptr(lse), None, None)


def attn_score(rows: Rows, q: torch.Tensor, k: Cache, lse: torch.Tensor, scores=None,
               n_slots: Optional[int] = None, scale: Optional[float] = None):
    """Full-attention selection scores [R, S] float32 (see sparse_attn_score);
    ``lse`` is the dense attention's [n_qsets, R, hq] log-normaliser."""
    L = load()
    if scores is None:
        scores = torch.empty(int(q.shape[1]), int(n_slots), dtype=torch.float32, device=q.device)
    _dense(scores, "scores", rows=True)
    d = score_desc(rows, q, k, lse, scale)
    _check(L.sparse_attn_score(ctypes.byref(d), _ptr(scores), int(scores.stride(0)), _stream()))
    return scores


# ---------------------------------------------------------------------------
# Prepared calls: descriptor and workspace built once, launch-only __call__
# ---------------------------------------------------------------------------


class Prepared:
    """A validated entry-point call whose descriptor (and workspace) are kept,
    so that each launch costs one ctypes call.  Every tensor the descriptor
    points to must stay alive as long as this object."""

    def __init__(self, fn_name: str, desc, op: int, device, keep=(), workspace=None):
        L = load()
        self.fn = getattr(L, fn_name)
        self.desc = desc
        self.ref = ctypes.byref(desc)
        need = int(L.sa_workspace_size(op, self.ref))
        if need == ctypes.c_size_t(-1).value:
            _check(-2)
        if need and workspace is not None and workspace.numel() >= need:
            # shared with calls that never overlap in time
            self.ws = workspace
        else:
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device) if need else None
        self.ws_ptr = _ptr(self.ws)
        self.need = need
        self.keep = keep

    def __call__(self, stream=None):
        _check(self.fn(self.ref, self.ws_ptr, self.need, _stream() if stream is None else stream))


def prepare_index_score(rows: Rows, q, w, k: Cache, scores, cand=None, cand_count=None,
                        skip_k: int = 0):
    d = index_desc(rows, q, w, k, scores, cand, cand_count, skip_k)
    return Prepared("sparse_index_score", d, SA_OP_INDEX_SCORE, q.device,
                    keep=(rows, q, w, k, scores, cand, cand_count))


def prepare_index_select(rows: Rows, q, w, kc: Cache, n_slots: int, k: int, idx, count,
                         cand=None, cand_count=None, block=0, max_blocks=0, pool=None,
                         pool_count=None, skip_k: int = 0, row_block: int = 0, workspace=None):
    """sparse_index_score with the fused selection: idx/count (and the pool)
    straight from the indexer, with n_slots score slots per row held in the
    workspace for row_block rows at a time (0 = all rows).  ``workspace``: a
    buffer to share with calls that never overlap in time, if large enough."""
    sel = topk_desc(rows, None, k, idx, count, cand, cand_count, block, max_blocks, pool,
                    pool_count)
    d = index_desc(rows, q, w, kc, None, cand, cand_count, skip_k, sel=sel, row_block=row_block,
                   n_slots=n_slots)
    return Prepared("sparse_index_score", d, SA_OP_INDEX_SCORE, q.device,
                    keep=(rows, q, w, kc, sel, idx, count, cand, cand_count, pool, pool_count),
                    workspace=workspace)


def prepare_topk_select(rows: Rows, scores, k, idx, count, cand=None, cand_count=None, block=0,
                        max_blocks=0, pool=None, pool_count=None, workspace=None):
    d = topk_desc(rows, scores, k, idx, count, cand, cand_count, block, max_blocks, pool,
                  pool_count)
    return Prepared("sparse_topk_select", d, SA_OP_TOPK_SELECT, scores.device,
                    keep=(rows, scores, idx, count, cand, cand_count, pool, pool_count),
                    workspace=workspace)


class PreparedScore:
    """A validated sparse_attn_score call, launch-only."""

    def __init__(self, rows: Rows, q, k: Cache, lse, scores, scale=None):
        L = load()
        self.fn = L.sparse_attn_score
        _dense(scores, "scores", rows=True)
        self.desc = score_desc(rows, q, k, lse, scale)
        self.ref = ctypes.byref(self.desc)
        self.scores_ptr = _ptr(scores)
        self.stride = int(scores.stride(0))
        self.keep = (rows, q, k, lse, scores)

    def __call__(self, stream=None):
        _check(self.fn(self.ref, self.scores_ptr, self.stride,
                       _stream() if stream is None else stream))


def prepare_attn_gather_fwd(rows: Rows, q, k: Cache, v: Optional[Cache], idx, count, o, lse=None,
                            scale=None, d_v=None, sink=None, gate=None):
    d = attn_desc(rows, q, k, v, idx, count, o, lse, scale, d_v, sink, gate)
    return Prepared("sparse_attn_gather_fwd", d, SA_OP_ATTN_GATHER_FWD, q.device,
                    keep=(rows, q, k, v, idx, count, o, lse, sink, gate))


# --------------------------------------------------------------------------
# Achievable peaks (include/sa_peak.h): what plain kernels reach on this GPU,
# for context next to the published peaks.


def _timed(launch, reps: int = 5) -> float:
    """Best of `reps` event-timed launches on the current stream, seconds."""
    best = float("inf")
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    return best


def peak_read_gbs(nbytes: int = 4 << 30, device="cuda") -> float:
    """HBM read rate (GB/s) of a streaming 16-byte-load kernel over `nbytes`
    (one contiguous slab per workgroup)."""
    L = load()
    src = torch.empty(nbytes, dtype=torch.uint8, device=device)
    src.fill_(1)
    grid = 1024  # four workgroups per CU, one contiguous slab each
    sink = torch.empty(grid * 256, dtype=torch.int32, device=device)
    launch = lambda: _check(L.sa_peak_read(_ptr(src), nbytes, _ptr(sink), grid, _stream()))
    launch()
    torch.cuda.synchronize()
    dt = _timed(launch)
    del src, sink
    return nbytes / dt / 1e9


def peak_mfma_tflops(dtype: str = "bf16", iters: int = 4096, device="cuda") -> float:
    """Dense MFMA rate (TFLOP/s) of a loop of independent 16x16 MFMA chains
    (bf16 16x16x32 or fp8 16x16x128) on every SIMD."""
    L = load()
    dt_code = {"bf16": 1, "fp8": 2}[dtype]
    grid = 256 * 4  # 4 workgroups of 4 waves per CU: 4 waves per SIMD
    sink = torch.empty(grid * 256, dtype=torch.float32, device=device)
    launch = lambda: _check(L.sa_peak_mfma(dt_code, iters, _ptr(sink), grid, _stream()))
    launch()
    torch.cuda.synchronize()
    dt = _timed(launch)
    flops = grid * 4 * iters * 8 * (16384 if dt_code == 1 else 65536)
    del sink
    return flops / dt / 1e12
