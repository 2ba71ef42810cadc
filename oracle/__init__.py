"""Python access to the CPU oracle (``oracle.c``), built with gcc into ``liboracle.so``.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the package's ``smoke()`` check
and the CPU-baseline leg of ``bench.py``.  The GPU product path never imports it.
It shares no code with that path; the only thing both sides use is the seeded
input generator in ``workloads``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test that plants a mistake in a copy of the oracle points this at the
# mutant's library (tests/test_oracle_mutants.py); nothing else sets it.
_LIB_OVERRIDE = os.environ.get("IDX_ORACLE_MUTANT_LIB")
_lib = None

Q_MXFP4 = 0
Q_FP8 = 1
SCORE_FP32 = 0
SCORE_BF16 = 1


def build() -> str:
    """Compile oracle.c (plain C, -O2, no FP contraction) into liboracle.so."""
    tmp = f"{_LIB}.tmp{os.getpid()}"   # concurrent builders never share a temporary
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            L = ctypes.CDLL(_LIB)
        d, i, i32p = ctypes.c_double, ctypes.c_int, ctypes.c_void_p
        for name in ("orc_e2m1", "orc_ue8m0", "orc_e4m3fn", "orc_bf16"):
            getattr(L, name).restype = d
            getattr(L, name).argtypes = [i]
        L.orc_round_bf16.restype = d
        L.orc_round_bf16.argtypes = [d]
        L.orc_candidate_tokens.restype = ctypes.c_int32
        L.orc_candidate_tokens.argtypes = [i32p, i, i, ctypes.c_int32, ctypes.c_int32, i32p]
        L.orc_expand_row.restype = ctypes.c_int32
        L.orc_expand_row.argtypes = [i32p, i, i, i, ctypes.c_int32, ctypes.c_int32, i32p,
                                     ctypes.c_int32, i32p]
        L.orc_select_topk.restype = ctypes.c_int32
        L.orc_select_topk.argtypes = [i32p, i32p, ctypes.c_int32, ctypes.c_int32, i32p]
        p, i64 = ctypes.c_void_p, ctypes.c_int64
        L.orc_indexer_rows.restype = i
        L.orc_indexer_rows.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p, i64, p, i64, p,
                                       i64, p, p, p, p, i64, p, ctypes.c_int32, p, i64, p, p, p,
                                       i64, p]
        L.orc_source_candidates.restype = i
        L.orc_source_candidates.argtypes = [i, i, i, i, i, i, i, p, p, p, p, p, p, i64, p, i64, p,
                                            i64, p, p, p, p, ctypes.c_int32, p, i64, p, i64]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def e2m1(code: int) -> float:
    return lib().orc_e2m1(int(code))


def ue8m0(b: int) -> float:
    return lib().orc_ue8m0(int(b))


def e4m3fn(b: int) -> float:
    return lib().orc_e4m3fn(int(b))


def bf16(code: int) -> float:
    return lib().orc_bf16(int(code))


def round_bf16(x: float) -> float:
    """x rounded to the nearest bf16 value (ties to even), as a float."""
    return lib().orc_round_bf16(float(x))


def candidate_tokens(cand_row, cbs: int, ks: int, ke: int) -> np.ndarray:
    cand_row = np.ascontiguousarray(cand_row, dtype=np.int32)
    out = np.empty(max(1, cand_row.size * cbs), dtype=np.int32)
    n = lib().orc_candidate_tokens(_ptr(cand_row), cand_row.size, cbs, ks, ke, _ptr(out))
    return out[:n].copy()


def expand_row(cand_row, cbs: int, sbk: int, ks: int, ke: int, nsb_cap: int):
    """(sparse_indices[nsb_cap], listed count, end) of one row."""
    cand_row = np.ascontiguousarray(cand_row, dtype=np.int32)
    out = np.empty(max(1, nsb_cap), dtype=np.int32)
    end = np.zeros(1, dtype=np.int32)
    n = lib().orc_expand_row(_ptr(cand_row), cand_row.size, cbs, sbk, ks, ke, _ptr(out),
                             nsb_cap, _ptr(end))
    return out[:nsb_cap].copy(), int(n), int(end[0])


def expand(case, sbk: int):
    """Schedule of every row of a case: (sparse_indices [R, NSB], end [R])."""
    s = case.spec
    nsb = s.nb * (s.cbs // sbk)
    si = np.empty((case.num_rows, nsb), dtype=np.int32)
    end = np.empty(case.num_rows, dtype=np.int32)
    for r in range(case.num_rows):
        si[r], _, end[r] = expand_row(case.candidate_blocks[r], s.cbs, sbk,
                                      int(case.row_ks[r]), int(case.row_ke[r]), nsb)
    return si, end


def select_topk(tokens, logits, topk: int) -> np.ndarray:
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    out = np.empty(max(1, topk), dtype=np.int32)
    lib().orc_select_topk(_ptr(tokens), _ptr(logits), tokens.size, topk, _ptr(out))
    return out[:topk].copy()


class RowResult:
    """Oracle output for a list of rows."""

    def __init__(self, rows, indices, tokens, logits, count, exact=None):
        self.rows = rows          # int32 [n]
        self.indices = indices    # int32 [n, topk]
        self.tokens = tokens      # int32 [n, cap] (first count[i] valid)
        self.logits = logits      # float32 [n, cap]
        self.count = count        # int32 [n]
        self.exact = exact        # float64 [n, cap]: the sums before the final rounding

    def row_tokens(self, i):
        return self.tokens[i, :self.count[i]]

    def row_logits(self, i):
        return self.logits[i, :self.count[i]]

    def row_exact(self, i):
        return self.exact[i, :self.count[i]]


def default_threads() -> int:
    """Host threads for oracle runs over many rows (at most 16)."""
    return max(1, min(16, os.cpu_count() or 1))


def indexer_rows(case, layer: int = 0, rows=None, q_format: str = "mxfp4", pool=None,
                 with_logits: bool = True, threads: int = 1,
                 score_format: str = "fp32") -> RowResult:
    """Run the oracle over the given rows (default: all) of one layer of a case.

    score_format "bf16": the layer's bf16 weights (LayerData.weights_bf16) and logits
    rounded to bf16 before the selection; "fp32": fp32 weights and logits.
    threads > 1 runs the same single-threaded C call on disjoint chunks of the rows
    at once (the C oracle keeps no state between calls and ctypes releases the GIL);
    each row's arithmetic is unchanged, only rows run side by side."""
    s = case.spec
    L = case.layers[layer]
    if rows is None:
        rows = np.arange(case.num_rows, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    if pool is None:
        pool = L.host_pool(s.page_bytes)
    pool = np.ascontiguousarray(pool)
    if threads > 1 and rows.size > 1:
        from concurrent.futures import ThreadPoolExecutor

        lib()   # load once, before the threads
        nchunk = min(rows.size, 4 * threads)
        chunks = [c for c in np.array_split(rows, nchunk) if c.size]
        with ThreadPoolExecutor(max_workers=threads) as ex:
            parts = list(ex.map(lambda c: indexer_rows(case, layer, c, q_format, pool,
                                                       with_logits, 1, score_format), chunks))

        def cat(f):
            return np.concatenate([getattr(p, f) for p in parts])

        return RowResult(rows, cat("indices"), cat("tokens") if with_logits else None,
                         cat("logits") if with_logits else None, cat("count"),
                         cat("exact") if with_logits else None)
    vb = s.values_bytes
    n = rows.size
    cap = max(1, s.nb * s.cbs)
    idx = np.empty((n, s.topk), dtype=np.int32)
    toks = np.empty((n, cap), dtype=np.int32) if with_logits else None
    lg = np.empty((n, cap), dtype=np.float32) if with_logits else None
    ex = np.empty((n, cap), dtype=np.float64) if with_logits else None
    cnt = np.empty(n, dtype=np.int32)
    fmt = Q_MXFP4 if q_format == "mxfp4" else Q_FP8
    if score_format == "bf16":
        sfmt, w = SCORE_BF16, np.ascontiguousarray(L.weights_bf16, dtype=np.uint16)
    else:
        sfmt, w = SCORE_FP32, np.ascontiguousarray(L.weights, dtype=np.float32)
    cand = np.ascontiguousarray(case.candidate_blocks, dtype=np.int32)
    bt = np.ascontiguousarray(case.block_table, dtype=np.int32)
    lib().orc_indexer_rows(
        s.num_heads, s.head_dim, s.page_size, s.cbs, s.nb, s.topk, fmt, sfmt,
        _ptr(L.q_values) if fmt == Q_MXFP4 else None,
        _ptr(L.q_scales) if fmt == Q_MXFP4 else None,
        _ptr(L.q_fp8) if fmt == Q_FP8 else None,
        _ptr(L.q_rowscale) if fmt == Q_FP8 else None,
        _ptr(w),
        _ptr(pool), s.page_bytes, pool.ctypes.data + vb, s.page_bytes,
        _ptr(bt), bt.shape[1],
        _ptr(case.row_ks), _ptr(case.row_ke), _ptr(case.row_table),
        _ptr(cand), cand.shape[1], _ptr(rows), n,
        _ptr(idx), s.topk, _ptr(toks), _ptr(lg), _ptr(ex), cap, _ptr(cnt))
    return RowResult(rows, idx, toks, lg, cnt, ex)


def gather_k_workspace(pool, page_size: int, head_dim: int, block_table, cu_seq_lens,
                       req_table=None, max_seq_len: int | None = None,
                       max_tokens: int | None = None, fill: int = 0):
    """The packed K workspace of a prefill chunk: the backend's gather of the chunk's
    paged K into one contiguous buffer before scoring (sparse_mqa_indexer page,
    _gather_prefill_chunk_k / cp_gather_indexer_k_quant_cache).  Request r's position p
    (p < cu[r+1] - cu[r], and p < max_seq_len) is copied to workspace row cu[r] + p
    (rows >= max_tokens are skipped): its D/2 value bytes and D/32 scale bytes, read
    through table row req_table[r] (r when None).  The page layout is the workload
    pool's: values [page_size][D/2] then scales [page_size][D/32].  A position whose
    table row, logical page or page id is out of range gets zeros; rows never written
    keep `fill`.  Returns (values [max_tokens, D/2], scales [max_tokens, D/32]) u8."""
    cu = np.asarray(cu_seq_lens, dtype=np.int64)
    bt = np.asarray(block_table)
    vrow, srow = head_dim // 2, head_dim // 32
    vbytes = page_size * vrow
    if max_tokens is None:
        max_tokens = int(cu[-1])
    if max_seq_len is None:
        max_seq_len = int(np.max(cu[1:] - cu[:-1], initial=0))
    values = np.full((max_tokens, vrow), fill, dtype=np.uint8)
    scales = np.full((max_tokens, srow), fill, dtype=np.uint8)
    for r in range(len(cu) - 1):
        tbl = int(req_table[r]) if req_table is not None else r
        if cu[r] < 0:
            continue
        for p in range(int(min(cu[r + 1] - cu[r], max_seq_len))):
            row = int(cu[r]) + p
            if row >= max_tokens:
                break
            lp, slot = p // page_size, p % page_size
            page = int(bt[tbl, lp]) if 0 <= tbl < bt.shape[0] and lp < bt.shape[1] else -1
            if 0 <= page < pool.shape[0]:
                values[row] = pool[page, slot * vrow:(slot + 1) * vrow]
                scales[row] = pool[page, vbytes + slot * srow:vbytes + (slot + 1) * srow]
            else:
                values[row] = 0
                scales[row] = 0
    return values, scales


def source_candidates(case, layer: int = 0, rows=None, nb: int | None = None,
                      q_format: str = "mxfp4", score_format: str = "fp32", pool=None,
                      threads: int = 1, score_width: int = 0):
    """The candidate-source layer's published pool for the given rows (default: all):
    (candidate_blocks int32 [n, nb], block scores float32 [n, score_width] or None).
    Block b of cbs = case.spec.cbs tokens scores the largest logit among its tokens in
    the row's [ks, ke) (NaN where it holds none); the row publishes the nb best blocks,
    ties toward the lower block id, ascending, then -1.  nb defaults to case.spec.nb."""
    s = case.spec
    L = case.layers[layer]
    nb = s.nb if nb is None else nb
    if rows is None:
        rows = np.arange(case.num_rows, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    if pool is None:
        pool = L.host_pool(s.page_bytes)
    pool = np.ascontiguousarray(pool)
    if threads > 1 and rows.size > 1:
        from concurrent.futures import ThreadPoolExecutor

        lib()
        chunks = [c for c in np.array_split(rows, min(rows.size, 4 * threads)) if c.size]
        with ThreadPoolExecutor(max_workers=threads) as ex:
            parts = list(ex.map(lambda c: source_candidates(case, layer, c, nb, q_format,
                                                            score_format, pool, 1, score_width),
                                chunks))
        return (np.concatenate([p[0] for p in parts]),
                np.concatenate([p[1] for p in parts]) if score_width else None)
    n = rows.size
    cand = np.empty((n, max(nb, 1)), dtype=np.int32)
    score = np.empty((n, score_width), dtype=np.float32) if score_width else None
    fmt = Q_MXFP4 if q_format == "mxfp4" else Q_FP8
    if score_format == "bf16":
        sfmt, w = SCORE_BF16, np.ascontiguousarray(L.weights_bf16, dtype=np.uint16)
    else:
        sfmt, w = SCORE_FP32, np.ascontiguousarray(L.weights, dtype=np.float32)
    bt = np.ascontiguousarray(case.block_table, dtype=np.int32)
    lib().orc_source_candidates(
        s.num_heads, s.head_dim, s.page_size, s.cbs, nb, fmt, sfmt,
        _ptr(L.q_values) if fmt == Q_MXFP4 else None,
        _ptr(L.q_scales) if fmt == Q_MXFP4 else None,
        _ptr(L.q_fp8) if fmt == Q_FP8 else None,
        _ptr(L.q_rowscale) if fmt == Q_FP8 else None,
        _ptr(w), _ptr(pool), s.page_bytes, pool.ctypes.data + s.values_bytes, s.page_bytes,
        _ptr(bt), bt.shape[1], _ptr(case.row_ks), _ptr(case.row_ke), _ptr(case.row_table),
        _ptr(rows), n, _ptr(cand), cand.shape[1], _ptr(score), score_width)
    return cand[:, :nb], score
