"""Seeded synthetic inputs for the candidate-consuming sparse MQA-logits indexer.

This module only *draws inputs*: context lengths, block tables, candidate blocks,
quantised Q/K codes with their scales, and per-head weights.  It contains none of
the indexer's arithmetic (no dequantisation, no dot product, no reduction, no
selection), so both the CPU oracle and the GPU path can consume its output
without sharing any computation.

Input model (stated once, used everywhere):

* MXFP4 tensors (Q and K): every element is the e2m1 code nearest to a draw of
  N(0, 1), packed two codes per byte with the even element in the low nibble; one
  UE8M0 scale byte ``127 + e`` per 32 consecutive elements, ``e`` uniform on the
  integers of ``scale_exp``.  The nearest-e2m1 code of a normal draw is sampled
  directly by inverse CDF from a uniform 32-bit word, which is the distribution
  of quantising a normal sample (to 2**-32 in probability) and far cheaper for
  the 1e9-element caches of the long-context workload.
* fp8 Q variant: x ~ N(0, 1) per element, one fp32 scale per row
  ``s_r = max|x_r| / 448``, codes = e4m3fn round-to-nearest-even of ``x / s_r``.
* weights: U(0, 1) / 8, fp32, one per (row, head).
* Decode rows of one request (``next_n`` > 1, MTP / speculative rows): the request's
  context end is drawn by ``ke_rule`` and row j of it ends j positions later; the
  request has one table row; with ``cand_rule="mtp_overlap"`` row 0 takes distinct
  random blocks and each later row keeps row 0's list but redraws each entry with
  probability ``mtp_resample`` from the blocks not yet listed.
* Paged K cache: pages of ``page_size`` tokens; a page holds the packed values
  ``[page_size][D/2]`` followed by the scale bytes ``[page_size][D/32]``.  The pool
  has ceil(1.25 x needed) pages; logical pages of every table row map to a random
  permutation of the pool (a fragmented cache); table entries past a row's last
  page are -1.  Only pages that hold a candidate block receive random contents
  (all referenced pages for ``fill="all"``); the rest stay zero and are never read
  by the sparse path.

Draw order for one case (fixed, so a (spec, seed) pair names the data exactly):
context ranges -> block table -> candidate blocks -> then per layer: Q (each
format in ``q_formats`` order) -> K pages -> weights.  K pages come in blocks of
256 pages, each from its own stream seeded by one draw of the main stream and
the block number, so they can be filled in parallel.
"""
from __future__ import annotations

import math
import statistics
from dataclasses import dataclass, field, replace
from functools import lru_cache

import numpy as np

GENERATOR_VERSION = 1

# e2m1 magnitudes in code order 0..7.  Used here only to *encode* normal draws
# into codes (the producer's side); nothing in this module decodes codes.
_E2M1_ENCODE_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_CHUNK = 1 << 20


@lru_cache(maxsize=None)
def _e2m1_sampler():
    """Tables that turn a uniform uint32 into the nearest-e2m1 code of a N(0,1) draw.

    The real line splits at the 15 points -m_j, 0, +m_j (m_j the midpoints of the
    e2m1 magnitude grid) into 16 intervals whose codes, left to right, are
    -6 .. -0, +0 .. +6.  A uniform u in [0, 2**32) falls into interval k when it
    passes k of the thresholds round(Phi(point) * 2**32): an inverse-CDF draw at
    2**-32 resolution.  A 2**16-entry table on the high half of u settles all but
    the 15 cells that straddle a threshold; those few are resolved exactly."""
    nd = statistics.NormalDist()
    grid = np.array(_E2M1_ENCODE_GRID)
    mids = ((grid[1:] + grid[:-1]) / 2.0).tolist()
    points = sorted([-m for m in mids] + [0.0] + mids)
    thresholds = np.array([round(nd.cdf(p) * 2 ** 32) for p in points], dtype=np.uint64)
    order_codes = np.array([15, 14, 13, 12, 11, 10, 9, 8, 0, 1, 2, 3, 4, 5, 6, 7], dtype=np.uint8)
    cell = np.arange(1 << 16, dtype=np.uint64) << 16
    lo = order_codes[np.searchsorted(thresholds, cell, side="right")]
    hi = order_codes[np.searchsorted(thresholds, cell | 0xFFFF, side="right")]
    return thresholds, order_codes, lo, lo != hi


def _e2m1_fill(rng: np.random.Generator, out: np.ndarray) -> None:
    """Fill the uint8 array ``out`` (any shape, C order) with packed e2m1 codes of
    N(0,1) draws: two codes per byte, the even element in the low nibble."""
    thresholds, order_codes, lut, straddle = _e2m1_sampler()
    flat = out.reshape(-1)
    n_codes = 2 * flat.size
    for s in range(0, n_codes, _CHUNK):
        m = min(_CHUNK, n_codes - s)
        u = rng.integers(0, 1 << 32, size=m, dtype=np.uint32)
        top = u >> 16
        c = lut[top]
        fix = np.nonzero(straddle[top])[0]
        if len(fix):
            c[fix] = order_codes[np.searchsorted(thresholds, u[fix].astype(np.uint64), side="right")]
        flat[s // 2:(s + m) // 2] = c[0::2] | (c[1::2] << 4)


def _e2m1_packed(rng: np.random.Generator, n_codes: int) -> np.ndarray:
    out = np.empty(n_codes // 2, dtype=np.uint8)
    _e2m1_fill(rng, out)
    return out


def _ue8m0_scales(rng: np.random.Generator, shape, exp_range) -> np.ndarray:
    lo, hi = exp_range
    return (127 + lo + rng.integers(0, hi - lo + 1, size=shape, dtype=np.uint32)).astype(np.uint8)


@dataclass(frozen=True)
class Spec:
    """Shape and structure of one synthetic workload."""

    name: str
    num_rows: int
    num_heads: int = 64
    head_dim: int = 128
    page_size: int = 64
    cbs: int = 64                     # candidate_block_size
    nb: int = 16                      # candidate blocks per row (columns of candidate_blocks)
    topk: int = 256
    layers: int = 1
    mode: str = "decode"              # decode: one table row per row; prefill: rows share table 0
    ke_rule: str = "fixed"            # fixed | uniform | uniform_unaligned | causal
    ke_lo: int = 4096
    ke_hi: int = 4096
    context: int = 0                  # prefill: positions held by the request's table
    ks_rule: str = "zero"             # zero | random
    cand_rule: str = "distinct"       # distinct | last_partial | causal_all | messy
    fill: str = "candidates"          # candidates | all
    q_formats: tuple = ("mxfp4",)     # subset of ("mxfp4", "fp8")
    scale_exp: tuple = (-4, 4)
    pool_factor: float = 1.25
    row_offset: int = 0               # prefill: position of row 0 in the request (causal ke = offset+i+1)
    next_n: int = 1                   # decode: rows per request (MTP / speculative rows) on one
                                      # table row; row j of a request has ke = the request's + j
    mtp_resample: float = 0.25        # cand_rule "mtp_overlap": share of row 0's blocks that
                                      # each later row of the request draws anew

    @property
    def page_bytes(self) -> int:
        return self.page_size * (self.head_dim // 2 + self.head_dim // 32)

    @property
    def values_bytes(self) -> int:
        return self.page_size * (self.head_dim // 2)


@dataclass
class LayerData:
    weights: np.ndarray                       # float32 [R, H]
    num_pages: int
    filled_pages: np.ndarray                  # int64 [n] physical page ids with contents
    filled_data: np.ndarray                   # uint8 [n, page_bytes]
    q_values: np.ndarray | None = None        # uint8 [R, H, D/2]  (mxfp4)
    q_scales: np.ndarray | None = None        # uint8 [R, H, D/32] (mxfp4)
    q_fp8: np.ndarray | None = None           # uint8 [R, H, D]    (e4m3fn codes)
    q_rowscale: np.ndarray | None = None      # float32 [R]

    @property
    def weights_bf16(self) -> np.ndarray:
        """The weights as bf16 codes (uint16 [R, H]): each fp32 weight rounded to the
        nearest bf16, ties to even (the producer's encoding of the bf16-weights variant;
        the weights are finite)."""
        u = np.ascontiguousarray(self.weights, dtype=np.float32).view(np.uint32)
        return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
                >> np.uint32(16)).astype(np.uint16)

    def host_pool(self, page_bytes: int) -> np.ndarray:
        """The whole page pool as one [num_pages, page_bytes] uint8 array.

        np.zeros is backed by lazily-committed zero pages, so a mostly-empty
        multi-GB pool costs only the pages that hold data."""
        pool = np.zeros((self.num_pages, page_bytes), dtype=np.uint8)
        if len(self.filled_pages):
            pool[self.filled_pages] = self.filled_data
        return pool


@dataclass
class Case:
    spec: Spec
    seed: int
    row_ks: np.ndarray            # int32 [R]
    row_ke: np.ndarray            # int32 [R]
    row_table: np.ndarray         # int32 [R] row -> block_table row
    block_table: np.ndarray       # int32 [T, P]
    candidate_blocks: np.ndarray  # int32 [R, NB]
    layers: list = field(default_factory=list)

    @property
    def num_rows(self) -> int:
        return self.spec.num_rows


def _draw_context(spec: Spec, rng: np.random.Generator):
    if spec.next_n > 1:
        # requests of next_n rows: the request's end drawn by the rule, row j one further
        n = spec.next_n
        if spec.mode != "decode" or spec.num_rows % n:
            raise ValueError("next_n > 1 needs decode rows in whole requests")
        ks_req, ke_req = _draw_context(replace(spec, num_rows=spec.num_rows // n, next_n=1), rng)
        j = np.arange(spec.num_rows) % n
        return np.repeat(ks_req, n), np.repeat(ke_req, n) + j
    R = spec.num_rows
    if spec.ke_rule == "fixed":
        ke = np.full(R, spec.ke_lo, dtype=np.int64)
    elif spec.ke_rule == "uniform":
        ke = rng.integers(spec.ke_lo, spec.ke_hi + 1, size=R)
    elif spec.ke_rule == "uniform_unaligned":
        ke = np.empty(R, dtype=np.int64)
        for r in range(R):
            v = int(rng.integers(spec.ke_lo, spec.ke_hi + 1))
            while v % spec.cbs == 0:
                v = int(rng.integers(spec.ke_lo, spec.ke_hi + 1))
            ke[r] = v
    elif spec.ke_rule == "causal":
        ke = spec.row_offset + np.arange(R, dtype=np.int64) + 1
    else:
        raise ValueError(spec.ke_rule)
    if spec.ks_rule == "zero":
        ks = np.zeros(R, dtype=np.int64)
    elif spec.ks_rule == "random":
        ks = np.array([int(rng.integers(0, int(k) + 1)) for k in ke], dtype=np.int64)
    else:
        raise ValueError(spec.ks_rule)
    return ks, ke


def _draw_block_table(spec: Spec, ke: np.ndarray, rng: np.random.Generator):
    ps = spec.page_size
    if spec.mode == "decode" and spec.next_n > 1:
        n = spec.next_n                           # one table row per request
        pages = [(int(ke[r + n - 1]) + ps - 1) // ps for r in range(0, spec.num_rows, n)]
        row_table = (np.arange(spec.num_rows) // n).astype(np.int32)
    elif spec.mode == "decode":
        pages = [(int(k) + ps - 1) // ps for k in ke]
        row_table = np.arange(spec.num_rows, dtype=np.int32)
    elif spec.mode == "prefill":
        ctx = max(spec.context, int(ke.max()) if len(ke) else 0)
        pages = [(ctx + ps - 1) // ps]
        row_table = np.zeros(spec.num_rows, dtype=np.int32)
    else:
        raise ValueError(spec.mode)
    needed = int(sum(pages))
    pool = max(1, math.ceil(spec.pool_factor * needed))
    perm = rng.permutation(pool)
    width = max(1, max(pages) if pages else 1)
    table = np.full((len(pages), width), -1, dtype=np.int32)
    pos = 0
    for i, n in enumerate(pages):
        table[i, :n] = perm[pos:pos + n]
        pos += n
    return table, row_table, pool


def _draw_candidates(spec: Spec, ks, ke, rng: np.random.Generator):
    R, nb, cbs = spec.num_rows, spec.nb, spec.cbs
    cand = np.full((R, nb), -1, dtype=np.int32)
    for r in range(R):
        k_end = int(ke[r])
        nblk = (k_end + cbs - 1) // cbs           # blocks that intersect [0, ke)
        if spec.cand_rule == "distinct":
            take = min(nb, nblk)
            ids = rng.choice(nblk, size=take, replace=False) if take else []
        elif spec.cand_rule == "last_partial":
            last = (k_end - 1) // cbs
            others = rng.choice(last, size=min(nb - 1, last), replace=False)
            ids = rng.permutation(np.concatenate([[last], others]))
        elif spec.cand_rule == "causal_all":
            if nblk <= nb:
                ids = rng.permutation(nblk)
            else:
                ids = rng.choice(nblk, size=nb, replace=False)
        elif spec.cand_rule == "mtp_overlap":
            # row 0 of a request: distinct random blocks; a later row keeps row 0's list
            # but draws each entry anew (from blocks not yet listed) with probability
            # mtp_resample
            take = min(nb, nblk)
            if r % spec.next_n == 0 or take == 0:
                ids = rng.choice(nblk, size=take, replace=False) if take else []
            else:
                ids = cand[r - r % spec.next_n][:take].astype(np.int64).copy()
                ids = ids[ids >= 0]
                redraw = rng.random(ids.size) < spec.mtp_resample
                free = np.setdiff1d(np.arange(nblk), ids)
                m = min(int(redraw.sum()), free.size)
                ids[np.nonzero(redraw)[0][:m]] = rng.choice(free, size=m, replace=False)
                ids = rng.permutation(ids)
        elif spec.cand_rule == "messy":
            # duplicates, -1/-2 padding and blocks past ke all appear
            ids = rng.integers(-2, nblk + 3, size=nb)
        else:
            raise ValueError(spec.cand_rule)
        ids = np.asarray(ids, dtype=np.int64)
        cand[r, :len(ids)] = ids
    return cand


def _pages_to_fill(spec: Spec, case_tables, row_table, ke, cand):
    ps, cbs = spec.page_size, spec.cbs
    table = case_tables
    if spec.fill == "all":
        ids = table[table >= 0]
        return np.unique(ids.astype(np.int64))
    out = []
    for r in range(spec.num_rows):
        trow = table[row_table[r]]
        npages = int((trow >= 0).sum())
        for b in cand[r]:
            if b < 0:
                continue
            lo = (int(b) * cbs) // ps
            hi = ((int(b) + 1) * cbs - 1) // ps
            for lp in range(lo, min(hi, npages - 1) + 1):
                out.append(int(trow[lp]))
    return np.unique(np.array(out, dtype=np.int64))


def _draw_q_mxfp4(spec: Spec, rng):
    R, H, D = spec.num_rows, spec.num_heads, spec.head_dim
    values = _e2m1_packed(rng, R * H * D).reshape(R, H, D // 2)
    scales = _ue8m0_scales(rng, (R, H, D // 32), spec.scale_exp)
    return values, scales


def _draw_q_fp8(spec: Spec, rng):
    import torch  # e4m3fn round-to-nearest-even encoding of the producer side

    R, H, D = spec.num_rows, spec.num_heads, spec.head_dim
    x = rng.standard_normal((R, H, D))
    amax = np.abs(x.reshape(R, -1)).max(axis=1)
    s = (amax / 448.0).astype(np.float32)
    s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    y = np.clip(x / s.astype(np.float64)[:, None, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, s


_PAGE_BLOCK = 256   # pages per independently seeded block of cache contents


def _draw_pages(spec: Spec, n: int, rng):
    """Contents of n cache pages: values then scales per page.

    The pages are drawn in blocks of _PAGE_BLOCK pages; block j uses its own PCG64
    stream seeded by (one 63-bit draw from ``rng``, j), so the result does not
    depend on how many threads fill the blocks."""
    from concurrent.futures import ThreadPoolExecutor
    import os

    ps, D = spec.page_size, spec.head_dim
    vb = ps * D // 2
    base = int(rng.integers(0, 1 << 63))
    out = np.empty((n, spec.page_bytes), dtype=np.uint8)

    def block(j):
        g = np.random.default_rng([base, j])
        lo, hi = j * _PAGE_BLOCK, min(n, (j + 1) * _PAGE_BLOCK)
        vals = np.empty((hi - lo, vb), dtype=np.uint8)
        _e2m1_fill(g, vals)
        out[lo:hi, :vb] = vals
        out[lo:hi, vb:] = _ue8m0_scales(g, (hi - lo, ps * D // 32), spec.scale_exp)

    nblocks = (n + _PAGE_BLOCK - 1) // _PAGE_BLOCK
    workers = max(1, min(8, os.cpu_count() or 1, nblocks))
    if workers == 1:
        for j in range(nblocks):
            block(j)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(block, range(nblocks)))
    return out


def generate(spec: Spec, seed: int = 0) -> Case:
    """Draw one case deterministically from (spec, seed) with numpy PCG64."""
    if spec.head_dim % 32:
        raise ValueError("head_dim must be a multiple of 32")
    rng = np.random.default_rng(seed)
    ks, ke = _draw_context(spec, rng)
    table, row_table, pool = _draw_block_table(spec, ke, rng)
    cand = _draw_candidates(spec, ks, ke, rng)
    fill = _pages_to_fill(spec, table, row_table, ke, cand)
    case = Case(spec=spec, seed=seed,
                row_ks=ks.astype(np.int32), row_ke=ke.astype(np.int32),
                row_table=row_table.astype(np.int32), block_table=table,
                candidate_blocks=cand)
    for _ in range(spec.layers):
        q = {}
        for fmt in spec.q_formats:
            if fmt == "mxfp4":
                q["q_values"], q["q_scales"] = _draw_q_mxfp4(spec, rng)
            elif fmt == "fp8":
                q["q_fp8"], q["q_rowscale"] = _draw_q_fp8(spec, rng)
            else:
                raise ValueError(fmt)
        data = _draw_pages(spec, len(fill), rng)
        w = (rng.random((spec.num_rows, spec.num_heads)) / 8.0).astype(np.float32)
        case.layers.append(LayerData(weights=w, num_pages=pool, filled_pages=fill,
                                     filled_data=data, **q))
    return case


# ---------------------------------------------------------------------------
# The five workloads of the method's evaluation (decode, ragged decode batch,
# causal prefill chunk, long-context multi-layer decode, sparse-vs-dense).
# ---------------------------------------------------------------------------
CONFIGS = {
    1: Spec(name="tiny_decode_r4_c1024_k256", num_rows=4, nb=16, topk=256,
            ke_rule="fixed", ke_lo=4096, ke_hi=4096, cand_rule="distinct"),
    2: Spec(name="decode_batch_r64_ctx8k-32k_c4096_k2048", num_rows=64, nb=64, topk=2048,
            ke_rule="uniform_unaligned", ke_lo=8192, ke_hi=32768, cand_rule="last_partial"),
    3: Spec(name="prefill_chunk_r4096_ctx8192_c64x64_k2048", num_rows=4096, nb=64, topk=2048,
            mode="prefill", ke_rule="causal", context=8192, cand_rule="causal_all"),
    4: Spec(name="long_decode_r256_ctx32k-128k_c8192_k2048_l4", num_rows=256, nb=128, topk=2048,
            layers=4, ke_rule="uniform", ke_lo=32768, ke_hi=131072, cand_rule="distinct"),
    5: Spec(name="sparse_vs_dense_r128_ctx64k_c4096_k2048", num_rows=128, nb=64, topk=2048,
            ke_rule="fixed", ke_lo=65536, ke_hi=65536, cand_rule="distinct", fill="all",
            q_formats=("mxfp4", "fp8")),
    # Beyond the five: decode with two rows per request (MTP / speculative rows on the
    # request's table row), the shape of the decode batch with 64 requests.
    6: Spec(name="mtp_decode_req64_n2_ctx8k-32k_c4096_k2048", num_rows=128, nb=64, topk=2048,
            ke_rule="uniform", ke_lo=8192, ke_hi=32768, cand_rule="mtp_overlap", next_n=2),
}


def config(n: int, **overrides) -> Spec:
    s = CONFIGS[n]
    return replace(s, **overrides) if overrides else s
