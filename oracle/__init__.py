"""fp64 CPU oracle for indexer-driven top-k sparse attention.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg call this; the GPU library never does, and this
module imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
independent rows).  This wrapper only builds it, converts torch CPU tensors to
raw buffers, and turns paged caches into logical entry order (the oracle reads
K/V by logical position; paging is a storage detail it never sees).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, E4M3, E2M1 = 0, 1, 2, 3

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.orc_decode_bf16.restype = ctypes.c_double
        L.orc_decode_bf16.argtypes = [ctypes.c_uint16]
        L.orc_decode_e4m3.restype = ctypes.c_double
        L.orc_decode_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_decode_e2m1.restype = ctypes.c_double
        L.orc_decode_e2m1.argtypes = [ctypes.c_uint8]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_n_avail.restype = i64
        L.orc_n_avail.argtypes = [ctypes.c_int, P, P, P, ctypes.c_int]
        L.orc_index_score.restype = ctypes.c_int
        L.orc_index_score.argtypes = [ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, P, i64, P, P,
                                      i64, P, i64]
        L.orc_topk_select.restype = ctypes.c_int
        L.orc_topk_select.argtypes = [ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int, P, i64, P,
                                      P, i64, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, P, P]
        L.orc_attention.restype = ctypes.c_int
        L.orc_attention.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, P, P, P,
                                    ctypes.c_int, i64, P, i64, P, f32, P, ctypes.c_int, P, P, P]
        L.orc_fa_score.restype = ctypes.c_int
        L.orc_fa_score.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P,
                                   i64, f32, P, i64]
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ---------------------------------------------------------------------------
# Buffer helpers
# ---------------------------------------------------------------------------


def _code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float8_e4m3fn:
        return E4M3
    raise TypeError("oracle: unsupported dtype %s" % t.dtype)


def _raw(t: torch.Tensor) -> np.ndarray:
    """Contiguous CPU bytes of ``t`` as a numpy array (no value conversion)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _i32(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def unpage(pool: torch.Tensor, block_table, page_size: int, n_seqs: int, cap: int) -> torch.Tensor:
    """Logical view [n_seqs, cap, ...] of a paged pool (CPU copy)."""
    pool = pool.detach()
    if block_table is None:
        return pool[:n_seqs, :cap].cpu().contiguous()
    bt = block_table.detach().to(pool.device).long()
    pages = -(-cap // page_size)
    out = pool[bt[:n_seqs, :pages]]  # [n_seqs, pages, page_size, ...]
    out = out.reshape(n_seqs, pages * page_size, *pool.shape[2:])
    return out[:, :cap].cpu().contiguous()


def n_avail(seq_of_row, pos_of_row, seq_len, stride: int) -> np.ndarray:
    so, po, sl = _i32(seq_of_row), _i32(pos_of_row), _i32(seq_len)
    L = lib()
    return np.array([L.orc_n_avail(r, _ptr(so), _ptr(po), _ptr(sl), stride)
                     for r in range(so.size)], dtype=np.int64)


# ---------------------------------------------------------------------------
# The three operations
# ---------------------------------------------------------------------------


def index_score(seq_of_row, pos_of_row, seq_len, stride: int, q: torch.Tensor, w: torch.Tensor,
                kidx: torch.Tensor, cand=None, cand_count=None) -> np.ndarray:
    """Scores [R, S] in float64.  ``kidx`` is logical [B, Lcap, D]; full mode
    gives S = Lcap, candidate mode S = cand.shape[1].  Slots outside the
    domain (or past cand_count) are NaN."""
    so, po, sl = _i32(seq_of_row), _i32(pos_of_row), _i32(seq_len)
    R = so.size
    H, D = int(q.shape[1]), int(q.shape[2])
    qa, ka = _raw(q), _raw(kidx)
    wa = np.ascontiguousarray(w.detach().cpu().float().numpy())
    Lcap = int(kidx.shape[1])
    ca = cc = None
    P = 0
    if cand is not None:
        ca, cc = _i32(cand), _i32(cand_count)
        P = int(ca.shape[1])
    S = P if cand is not None else Lcap
    out = np.empty((R, S), dtype=np.float64)
    rc = lib().orc_index_score(R, _ptr(so), _ptr(po), _ptr(sl), stride, H, D, _code(q), _ptr(qa),
                               _ptr(wa), _code(kidx), _ptr(ka), Lcap, _ptr(ca), _ptr(cc), P,
                               _ptr(out), S)
    if rc != 0:
        raise ValueError("orc_index_score failed (%d)" % rc)
    return out


def topk_select(seq_of_row, pos_of_row, seq_len, stride: int, window: int, scores: np.ndarray,
                k: int, cand=None, cand_count=None, block: int = 0, max_blocks: int = 0):
    """Returns (idx [R, k] int32, count [R]) and, if block > 0,
    (pool [R, max_blocks*block], pool_count [R])."""
    so, po, sl = _i32(seq_of_row), _i32(pos_of_row), _i32(seq_len)
    R = so.size
    sc = np.ascontiguousarray(scores, dtype=np.float64)
    S = int(sc.shape[1])
    ca = cc = None
    P = 0
    if cand is not None:
        ca, cc = _i32(cand), _i32(cand_count)
        P = int(ca.shape[1])
        assert P == S
    idx = np.full((R, max(k, 1)), -1, dtype=np.int32)
    cnt = np.zeros(R, dtype=np.int32)
    pool = pcnt = None
    if block > 0:
        pool = np.full((R, max_blocks * block), -1, dtype=np.int32)
        pcnt = np.zeros(R, dtype=np.int32)
    rc = lib().orc_topk_select(R, _ptr(so), _ptr(po), _ptr(sl), stride, window, _ptr(sc), S,
                               _ptr(ca), _ptr(cc), P, k, _ptr(idx), _ptr(cnt), block, max_blocks,
                               _ptr(pool), _ptr(pcnt))
    if rc != 0:
        raise ValueError("orc_topk_select failed (%d)" % rc)
    if block > 0:
        return idx[:, :k], cnt, pool, pcnt
    return idx[:, :k], cnt


def attention(seq_of_row, pos_of_row, seq_len, stride: int, window: int, q: torch.Tensor,
              K: torch.Tensor, V=None, idx=None, count=None, scale: float = None, hkv: int = None,
              k_scale: torch.Tensor = None, v_scale: torch.Tensor = None, v_from_k: bool = False,
              dv: int = None, fp4: bool = False, sink=None, gate: torch.Tensor = None):
    """Joint softmax over window + selected positions (``sink`` [n_sets, Hq]
    and ``gate`` [n_sets, R, Hq, dv]: the optional sink bias and output gate).

    q [n_sets, R, Hq, dqk]; K logical [B, Lcap, Hkv, dqk] (or FP4 codes
    [B, Lcap, Hkv, dqk/2] uint8 with ``k_scale`` [B, Lcap, Hkv, dqk/16]).
    Returns (o [n_sets, R, Hq, dv] float64, lse [n_sets, R, Hq] float64)."""
    so, po, sl = _i32(seq_of_row), _i32(pos_of_row), _i32(seq_len)
    n_sets, R, Hq, dqk = (int(x) for x in q.shape)
    Hkv = int(K.shape[2]) if hkv is None else hkv
    if dv is None:
        dv = int(V.shape[3]) if V is not None else dqk
    Lcap = int(K.shape[1])
    qa = _raw(q)
    if fp4:
        kd = E2M1
        ka = np.ascontiguousarray(K.detach().cpu().numpy().astype(np.uint8))
        ksa = np.ascontiguousarray(k_scale.detach().cpu().numpy().astype(np.uint8))
        va = vsa = None
        if not v_from_k:
            va = np.ascontiguousarray(V.detach().cpu().numpy().astype(np.uint8))
            vsa = np.ascontiguousarray(v_scale.detach().cpu().numpy().astype(np.uint8))
    else:
        kd = _code(K)
        ka = _raw(K)
        ksa = vsa = None
        va = None if v_from_k else _raw(V)
    ia = ca = None
    istride = 0
    if idx is not None:
        ia, ca = _i32(idx), _i32(count)
        istride = int(ia.shape[1])
    if scale is None:
        scale = 1.0 / float(np.sqrt(dqk))
    o = np.empty((n_sets, R, Hq, dv), dtype=np.float64)
    lse = np.empty((n_sets, R, Hq), dtype=np.float64)
    sa = None
    if sink is not None:
        sink = sink.detach().cpu() if isinstance(sink, torch.Tensor) else torch.as_tensor(sink)
        sa = np.ascontiguousarray(sink.float().numpy().reshape(n_sets, Hq))
    ga, gd = None, F32
    if gate is not None:
        ga, gd = _raw(gate), _code(gate)
    rc = lib().orc_attention(n_sets, R, _ptr(so), _ptr(po), _ptr(sl), stride, window, Hq, Hkv, dqk,
                             dv, _code(q), _ptr(qa), kd, _ptr(ka), _ptr(ksa), _ptr(va), _ptr(vsa),
                             1 if v_from_k else 0, Lcap, _ptr(ia), istride, _ptr(ca),
                             ctypes.c_float(scale), _ptr(sa), gd, _ptr(ga), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("orc_attention failed (%d)" % rc)
    return o, lse


def fa_score(seq_of_row, pos_of_row, seq_len, stride: int, q: torch.Tensor, K: torch.Tensor,
             scale: float = None) -> np.ndarray:
    """Full-attention selection scores [R, Lcap] in float64: for every visible
    entry, the dense-attention probability each query head (of every query
    set) gives it, summed over the heads; NaN outside the domain.  q
    [n_sets, R, Hq, dqk]; K logical [B, Lcap, Hkv, dqk]."""
    so, po, sl = _i32(seq_of_row), _i32(pos_of_row), _i32(seq_len)
    n_sets, R, Hq, dqk = (int(x) for x in q.shape)
    Hkv, Lcap = int(K.shape[2]), int(K.shape[1])
    if scale is None:
        scale = 1.0 / float(np.sqrt(dqk))
    out = np.empty((R, Lcap), dtype=np.float64)
    rc = lib().orc_fa_score(n_sets, R, _ptr(so), _ptr(po), _ptr(sl), stride, Hq, Hkv, dqk,
                            _code(q), _ptr(_raw(q)), _code(K), _ptr(_raw(K)), Lcap,
                            ctypes.c_float(scale), _ptr(out), Lcap)
    if rc != 0:
        raise ValueError("orc_fa_score failed (%d)" % rc)
    return out


def decode_bf16(bits: int) -> float:
    return float(lib().orc_decode_bf16(bits))


def decode_e4m3(bits: int) -> float:
    return float(lib().orc_decode_e4m3(bits))


def decode_e2m1(bits: int) -> float:
    return float(lib().orc_decode_e2m1(bits))
