"""Seeded synthetic inputs for indexer-driven top-k sparse attention.

This module only draws random tensors and lays them out; it holds none of the
method's arithmetic (no scoring, selection, softmax or decoding).  Both the GPU
path and the CPU oracle are fed from here.

Every tensor is drawn from its own stream, ``torch.Generator`` seeded with
``1000 * config + slot``, on the device the caller names.  The same seed on the
same device type gives the same tensor.  Large inputs are drawn on the GPU and
the oracle receives copies of exactly the slices it needs.

Workload shapes follow the five configurations the method is measured on:

* ``tiny``     -- 1 sequence of 512 tokens, every row a query, fp32;
* ``hysparse2`` -- HySparse2-style decode: 32 sequences x 32768 tokens, window
  128 + top-1024 from one shared paged KV (64-token pages), 8 KV heads of 128,
  64 query heads, 6 query sets (1 FA + 5 SA) reusing one index tensor;
* ``dsa``      -- DSA-style prefill: 65536 causal rows, FP8 indexer 64x128,
  top-2048, MLA latent KV 576 wide (V = first 512), 128 query heads;
* ``csa``      -- CSA-style decode over entries compressed at stride 4;
* ``csa2``     -- CSA2 hierarchical decode with an FP4 (E2M1 + E4M3/16) KV;
* ``hca``      -- HCA decode: every entry compressed at stride 128, read
  densely (no selector);
* ``csa2_prefill`` -- the CSA2 layer group (Full + pool, Reindex) over every
  token of a 131072-token prefill at stride 4.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional

import torch

# ---------------------------------------------------------------------------
# Random streams
# ---------------------------------------------------------------------------

_CHUNK = 1 << 26  # elements drawn per call, to bound temporaries


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def normal(shape, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """N(0, 1) in float32, rounded (round-to-nearest-even) to ``dtype``."""
    g = _gen(device, seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for lo in range(0, flat.numel(), _CHUNK):
        hi = min(flat.numel(), lo + _CHUNK)
        flat[lo:hi] = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32).to(dtype)
    return out


def uniform01(shape, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(device, seed)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def small_ints(shape, seed: int, device="cpu", dtype=torch.float32, lo=-4, hi=4) -> torch.Tensor:
    """Uniform integers in [lo, hi], stored exactly in ``dtype``."""
    g = _gen(device, seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for a in range(0, flat.numel(), _CHUNK):
        b = min(flat.numel(), a + _CHUNK)
        flat[a:b] = torch.randint(lo, hi + 1, (b - a,), generator=g, device=device).to(dtype)
    return out


def permutation(n: int, seed: int, device="cpu") -> torch.Tensor:
    g = _gen("cpu", seed)
    return torch.randperm(n, generator=g).to(device=device, dtype=torch.int32)


# ---------------------------------------------------------------------------
# FP4 E2M1 + E4M3-per-16-channel encoding of generated values (input
# generation only: the GPU path and the oracle both consume the stored codes)
# ---------------------------------------------------------------------------

# Magnitudes representable in E2M1, by 3-bit code.
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _e2m1_code(mag: torch.Tensor) -> torch.Tensor:
    """Round non-negative magnitudes to the nearest E2M1 grid value, ties to the
    even code, saturating at 6; returns the 3-bit magnitude code."""
    grid = torch.tensor(_E2M1_GRID, dtype=torch.float32, device=mag.device)
    mids = (grid[1:] + grid[:-1]) * 0.5
    code = torch.bucketize(mag, mids)  # index of the first midpoint >= mag
    # bucketize puts a value equal to a midpoint in the lower bucket; move odd
    # lower codes up so exact ties go to the even code.
    tie = (code < 7) & (mag == mids[code.clamp(max=6)])
    code = torch.where(tie & (code % 2 == 1), code + 1, code)
    return code.to(torch.uint8)


def fp4_encode(x: torch.Tensor):
    """Quantise ``x[..., d]`` (d a multiple of 16) to E2M1 codes with one E4M3
    scale per 16 channels: scale = e4m3(amax / 6), code = e2m1(x / scale).
    Returns (codes uint8 [..., d/2] with the even channel in the low nibble,
    scales uint8 [..., d/16] holding E4M3 bit patterns)."""
    d = x.shape[-1]
    assert d % 16 == 0
    xf = x.float().reshape(*x.shape[:-1], d // 16, 16)
    amax = xf.abs().amax(dim=-1, keepdim=True)
    scale8 = (amax / 6.0).to(torch.float8_e4m3fn)
    scale = scale8.float()
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    y = torch.where(scale > 0, xf / safe, torch.zeros_like(xf))
    code = _e2m1_code(y.abs().clamp(max=6.0))
    code = code | ((y < 0).to(torch.uint8) << 3)
    code = code.reshape(*x.shape[:-1], d)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), scale8.view(torch.uint8).reshape(*x.shape[:-1], d // 16).contiguous()


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------


@dataclass
class Workload:
    """One configuration of the path.  Sizes are in tokens unless named
    otherwise.  ``stride`` is the number of tokens per cache entry."""

    name: str
    cfg_id: int
    n_seqs: int
    seq_len: int
    prefill: bool  # True: every token of sequence 0 is a query row
    stride: int
    window: int
    k: int
    idx_heads: int
    idx_dim: int
    idx_dtype: torch.dtype
    hq: int
    hkv: int
    dqk: int
    dv: int
    kv_mode: str  # "separate" (K and V rows), "shared" (V = first dv of K), "fp4" (shared, E2M1)
    attn_dtype: torch.dtype
    n_qsets: int
    page_size: int  # 0 = contiguous per sequence
    block: int = 0  # block-max pool block (0 = none)
    max_blocks: int = 0
    n_reuse: int = 0  # extra query sets that reuse the Reindex indices
    tail_variant: bool = False  # sequence b loses (b mod 4) tokens
    w_signed_ints: bool = True  # integer variant: w in [-4, 4]
    seq_lens_override: Optional[tuple] = None

    def seq_lens(self):
        if self.seq_lens_override is not None:
            return list(self.seq_lens_override)
        if self.tail_variant:
            return [self.seq_len - (b % 4) for b in range(self.n_seqs)]
        return [self.seq_len] * self.n_seqs

    @property
    def n_entries_cap(self) -> int:
        """Cache capacity in entries per sequence."""
        lcap = max(self.seq_lens()) // self.stride
        if self.page_size:
            lcap = -(-lcap // self.page_size) * self.page_size
        return lcap

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY = Workload("tiny", 0, n_seqs=1, seq_len=512, prefill=True, stride=1, window=32, k=64,
                idx_heads=4, idx_dim=64, idx_dtype=torch.float32, hq=8, hkv=1, dqk=64, dv=64,
                kv_mode="separate", attn_dtype=torch.float32, n_qsets=1, page_size=16)
HYSPARSE2 = Workload("hysparse2", 1, n_seqs=32, seq_len=32768, prefill=False, stride=1, window=128,
                     k=1024, idx_heads=16, idx_dim=64, idx_dtype=torch.bfloat16, hq=64, hkv=8,
                     dqk=128, dv=128, kv_mode="separate", attn_dtype=torch.bfloat16, n_qsets=6,
                     page_size=64)
DSA = Workload("dsa", 2, n_seqs=1, seq_len=65536, prefill=True, stride=1, window=0, k=2048,
               idx_heads=64, idx_dim=128, idx_dtype=torch.float8_e4m3fn, hq=128, hkv=1, dqk=576,
               dv=512, kv_mode="shared", attn_dtype=torch.bfloat16, n_qsets=1, page_size=64)
CSA = Workload("csa", 3, n_seqs=16, seq_len=131072, prefill=False, stride=4, window=0, k=512,
               idx_heads=32, idx_dim=128, idx_dtype=torch.bfloat16, hq=64, hkv=1, dqk=512, dv=512,
               kv_mode="shared", attn_dtype=torch.bfloat16, n_qsets=1, page_size=0)
CSA2 = Workload("csa2", 4, n_seqs=8, seq_len=262144, prefill=False, stride=1, window=0, k=512,
                idx_heads=32, idx_dim=128, idx_dtype=torch.bfloat16, hq=64, hkv=1, dqk=512, dv=512,
                kv_mode="fp4", attn_dtype=torch.bfloat16, n_qsets=1, page_size=0, block=8,
                max_blocks=2048, n_reuse=3)

# HCA: heavily compressed entries (one per 128 tokens) read densely with no
# selector ("CSA, HCA and CSA2", sections 1.2 and 6.2: HCA attends to every
# entry of the shorter sequence; 8192 entries at 1M tokens).
HCA = Workload("hca", 5, n_seqs=16, seq_len=1048576, prefill=False, stride=128, window=8192, k=0,
               idx_heads=0, idx_dim=0, idx_dtype=torch.bfloat16, hq=64, hkv=1, dqk=512, dv=512,
               kv_mode="shared", attn_dtype=torch.bfloat16, n_qsets=1, page_size=0)

# CSA2's hierarchical indexer in prefill ("CSA, HCA and CSA2", section 3.1,
# the layer-group cost breakdown: n = 131072 tokens at m = 4 give 32768
# entries; the Full layer builds a 4096-entry pool, the Reindex layer keeps
# 1024; section 2.2: prefill must not materialise an n x n_c score or pool).
# Every token is a query row; the FP8 indexer runs as the row-block GEMM.
CSA2_PREFILL = Workload("csa2_prefill", 6, n_seqs=1, seq_len=131072, prefill=True, stride=4,
                        window=0, k=1024, idx_heads=32, idx_dim=128,
                        idx_dtype=torch.float8_e4m3fn, hq=64, hkv=1, dqk=512, dv=512,
                        kv_mode="shared", attn_dtype=torch.bfloat16, n_qsets=1, page_size=0,
                        block=8, max_blocks=512, n_reuse=0)

WORKLOADS = {w.name: w for w in (TINY, HYSPARSE2, DSA, CSA, CSA2, HCA, CSA2_PREFILL)}


# ---------------------------------------------------------------------------
# Problem instances
# ---------------------------------------------------------------------------


@dataclass
class Cache:
    """Rows of a cache, paged: logical entry e of sequence b lives in
    ``pool[block_table[b, e // page_size], e % page_size]``.  With no block
    table the pool is ``[n_seqs, cap, ...]`` contiguous."""

    pool: torch.Tensor
    block_table: Optional[torch.Tensor]
    page_size: int
    scale: Optional[torch.Tensor] = None  # FP4 only: E4M3 scale bytes, same leading layout


@dataclass
class Problem:
    wl: Workload
    integer: bool
    seq_of_row: torch.Tensor
    pos_of_row: torch.Tensor
    seq_len: torch.Tensor
    idx_q: list  # one [R, H_I, d_I] tensor per indexer layer (Full, then Reindex)
    idx_w: list  # matching [R, H_I] float32
    kidx: Cache
    q: list  # one [n_sets, R, Hq, dqk] tensor per attention call
    k: Cache
    v: Optional[Cache]
    extra: dict = field(default_factory=dict)

    @property
    def n_rows(self) -> int:
        return int(self.seq_of_row.numel())


def _paged_shape(n_seqs, cap_entries, page_size):
    if page_size:
        max_pages = -(-cap_entries // page_size)
        return n_seqs * max_pages, max_pages
    return None, None


def _block_table(n_seqs, max_pages, seed, device):
    perm = permutation(n_seqs * max_pages, seed, device="cpu")
    return perm.view(n_seqs, max_pages).to(device)


def _draw(shape, seed, device, dtype, integer, kind="normal"):
    if integer:
        return small_ints(shape, seed, device=device, dtype=dtype)
    if kind == "uniform":
        return uniform01(shape, seed, device=device).to(dtype)
    return normal(shape, seed, device=device, dtype=dtype)


def make_problem(wl: Workload, device="cpu", integer=False, seed_base=None,
                 rows: Optional[list] = None) -> Problem:
    """Draw every input of workload ``wl`` on ``device``.

    ``integer=True`` gives the integer-valued variant: indexer q, k and w are
    uniform integers in [-4, 4] (every score then is an exact integer in
    float32, so selections can be compared bit for bit); attention inputs stay
    N(0, 1).  ``rows`` restricts the
    query rows of a prefill workload to the listed positions of sequence 0.
    """
    base = 1000 * (wl.cfg_id + 1) if seed_base is None else seed_base
    B = wl.n_seqs
    lens = wl.seq_lens()
    seq_len = torch.tensor(lens, dtype=torch.int32)
    if wl.prefill:
        pos = list(range(lens[0])) if rows is None else list(rows)
        seq_of_row = torch.zeros(len(pos), dtype=torch.int32)
        pos_of_row = torch.tensor(pos, dtype=torch.int32)
    else:
        seq_of_row = torch.arange(B, dtype=torch.int32)
        pos_of_row = seq_len - 1
    R = int(seq_of_row.numel())
    cap = wl.n_entries_cap

    # --- indexer inputs (none when k = 0: the window covers every entry) ------
    n_idx_layers = 0 if wl.k == 0 else (2 if wl.block else 1)
    idx_q, idx_w = [], []
    for layer in range(n_idx_layers):
        idx_q.append(_draw((R, wl.idx_heads, wl.idx_dim), base + 1 + 10 * layer, device,
                           wl.idx_dtype, integer))
        if integer:
            idx_w.append(small_ints((R, wl.idx_heads), base + 2 + 10 * layer, device=device,
                                    lo=-4 if wl.w_signed_ints else 0))
        else:
            idx_w.append(uniform01((R, wl.idx_heads), base + 2 + 10 * layer, device=device))

    n_pages, max_pages = _paged_shape(B, cap, wl.page_size)
    bt = _block_table(B, max_pages, base + 7, device) if wl.page_size else None
    kidx = None
    if n_idx_layers and wl.page_size:
        kpool = _draw((n_pages, wl.page_size, wl.idx_dim), base + 3, device, wl.idx_dtype, integer)
        kidx = Cache(kpool, bt, wl.page_size)
    elif n_idx_layers:
        kpool = _draw((B, cap, wl.idx_dim), base + 3, device, wl.idx_dtype, integer)
        kidx = Cache(kpool, None, 0)

    # --- attention inputs ---------------------------------------------------
    n_calls = 2 if wl.block else 1
    q = []
    for call in range(n_calls):
        sets = wl.n_qsets if call == 0 else 1 + wl.n_reuse
        q.append(_draw((sets, R, wl.hq, wl.dqk), base + 4 + 10 * call, device, wl.attn_dtype,
                       False))
    lead = (n_pages, wl.page_size) if wl.page_size else (B, cap)
    if wl.kv_mode == "fp4":
        x = _draw(lead + (wl.hkv, wl.dqk), base + 5, device, torch.float32, False)
        codes, scales = fp4_encode(x)
        del x
        kc = Cache(codes, bt, wl.page_size, scale=scales)
        vc = None
    else:
        kc = Cache(_draw(lead + (wl.hkv, wl.dqk), base + 5, device, wl.attn_dtype, False), bt,
                   wl.page_size)
        vc = None
        if wl.kv_mode == "separate":
            vc = Cache(_draw(lead + (wl.hkv, wl.dv), base + 6, device, wl.attn_dtype, False), bt,
                       wl.page_size)
    return Problem(wl, integer, seq_of_row.to(device), pos_of_row.to(device), seq_len.to(device),
                   idx_q, idx_w, kidx, q, kc, vc)


def small_version(wl: Workload, **kw) -> Workload:
    """A reduced-size copy of ``wl`` for oracle-speed parity cases: the same
    head counts, widths and dtypes, fewer and shorter sequences."""
    return wl.replace(**kw)
