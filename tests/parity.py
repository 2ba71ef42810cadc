"""Helpers that run the HIP path through the C ABI and compare it with the oracle.

Floating point: |gpu - oracle| <= 1e-6 + 1e-5 * |oracle| for every candidate token
(with signed head weights, 1e-5 * sum_h |w_h| ReLU(s_h) in place of |oracle|: the
same bound when no weight is negative).
Indices: with theta the oracle's count-th selected logit and tau = 1e-6 + 1e-5*|theta|,
the GPU picks exactly count distinct valid tokens in ascending order, every token
with oracle logit > theta + tau, none with oracle logit < theta - tau, -1 in the
other slots, and exactly the oracle's set when no other oracle logit lies within
tau of theta.  The GPU's selection is also checked bit-exactly against its own
logits (an independent lexsort here), which pins the top-k kernel without any
rounding slack.
"""
from __future__ import annotations

import numpy as np

ATOL = 1e-6
RTOL = 1e-5


def gpu_row_tokens(si_row, kept, sbk, ks, ke, logits_row):
    """(tokens, logits) of a row's valid sparse columns, ascending by token."""
    cols = np.arange(kept * sbk)
    toks = si_row[cols // sbk].astype(np.int64) * sbk + cols % sbk
    ok = (toks >= ks) & (toks < ke)
    return toks[ok].astype(np.int32), logits_row[cols[ok]]


def exact_topk(tokens, logits, topk):
    """Top-k of (tokens, fp32 logits): larger logit first, ties to the lower token."""
    lg = logits.astype(np.float32) + np.float32(0.0)     # -0 -> +0
    order = np.lexsort((tokens, -lg.astype(np.float64)))
    count = min(topk, tokens.size)
    out = np.full(topk, -1, np.int32)
    out[:count] = np.sort(tokens[order[:count]])
    return out


def check_logits(o_tokens, o_logits, g_tokens, g_logits, what="", o_scale=None):
    """o_scale (optional): per token sum_h |w_h| * ReLU(s_h), the oracle run with |w|;
    the relative tolerance applies to it instead of |logit| (the two are equal when no
    weight is negative; with signed weights the terms cancel, and a sum's rounding
    error scales with the magnitudes of its terms, not with the result)."""
    np.testing.assert_array_equal(g_tokens, o_tokens, err_msg=f"{what}: candidate tokens differ")
    g64, o64 = g_logits.astype(np.float64), o_logits.astype(np.float64)
    same = g64 == o64                     # also equal infinities (overflowed sums)
    with np.errstate(invalid="ignore"):
        err = np.where(same, 0.0, np.abs(g64 - o64))
    err[np.isnan(err)] = np.inf           # a NaN on either side never matches
    mag = np.abs(o64) if o_scale is None else o_scale.astype(np.float64)
    lim = ATOL + RTOL * np.where(np.isfinite(mag), mag, 0.0)
    bad = np.nonzero(err > lim)[0]
    assert bad.size == 0, (f"{what}: {bad.size} logits outside tolerance, first token "
                           f"{o_tokens[bad[0]]}: gpu {g_logits[bad[0]]!r} oracle {o_logits[bad[0]]!r}")


def check_indices(o_tokens, o_logits, o_idx, g_idx, topk, what="", o_scale=None):
    n = o_tokens.size
    count = min(topk, n)
    assert np.all(g_idx[count:] == -1), f"{what}: slots past count={count} are not -1"
    chosen = g_idx[:count]
    assert np.all(np.diff(chosen) > 0), f"{what}: chosen ids not strictly ascending"
    if count == 0:
        return
    pos = np.searchsorted(o_tokens, chosen)
    assert np.all(pos < n) and np.all(o_tokens[np.minimum(pos, n - 1)] == chosen), \
        f"{what}: a chosen id is not a valid candidate token"
    ol = o_logits.astype(np.float64)
    o_sel = np.isin(o_tokens, o_idx[:count])
    theta = ol[o_sel].min()
    if not np.isfinite(theta):
        # the count-th logit is -inf: every finite logit is taken and the -inf ones go
        # by token order, so the set is exact
        np.testing.assert_array_equal(chosen, o_idx[:count], err_msg=f"{what}: set differs")
        return
    # with o_scale (signed weights), the largest magnitude of the row bounds every
    # logit's error
    fin = o_scale[np.isfinite(o_scale)] if o_scale is not None else None
    tau = ATOL + RTOL * (abs(theta) if o_scale is None else float(np.max(fin, initial=0.0)))
    g_sel = np.zeros(n, bool)
    g_sel[pos] = True
    must = ol > theta + tau
    assert np.all(g_sel[must]), f"{what}: missed {np.count_nonzero(must & ~g_sel)} clear winners"
    forbid = ol < theta - tau
    assert not np.any(g_sel & forbid), f"{what}: picked {np.count_nonzero(g_sel & forbid)} clear losers"
    if np.count_nonzero(np.abs(ol - theta) <= tau) == 1:
        np.testing.assert_array_equal(chosen, o_idx[:count], err_msg=f"{what}: set differs")


def check_topk_exact_for_own_logits(g_tokens, g_logits, g_idx, topk, what=""):
    np.testing.assert_array_equal(g_idx, exact_topk(g_tokens, g_logits, topk),
                                  err_msg=f"{what}: GPU top-k is not exact for its own logits")


def round_bf16_np(x):
    """float64 array -> the nearest bf16 values (ties to even) as float64: spacing
    2^(e-8) on [2^(e-1), 2^e), 2^-133 below 2^-126, infinity from 2^128 on (numpy's rint
    rounds halves to even)."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)
    lsb = np.maximum(e - 8, -133)
    v = np.ldexp(np.rint(np.ldexp(a, -lsb)), lsb)
    v = np.where(v >= 2.0 ** 128, np.inf, v)
    v = np.where(np.isfinite(a), v, a)
    return np.copysign(v, x)


def check_logits_bf16(o_tokens, o_exact, o_logits, g_tokens, g_logits, what=""):
    """bf16 scoring: each GPU logit is a bf16 value (low 16 bits zero) that rounds some
    value within the fp32 tolerance of the oracle's exact sum: between the roundings of
    exact - tol and exact + tol (rounding is monotone), so it equals the oracle's bf16
    logit except where the exact sum lies within tol of a rounding midpoint."""
    np.testing.assert_array_equal(g_tokens, o_tokens, err_msg=f"{what}: candidate tokens differ")
    assert np.all((g_logits.view(np.uint32) & 0xFFFF) == 0), f"{what}: a logit is not a bf16 value"
    tol = ATOL + RTOL * np.abs(o_exact)
    lo, hi = round_bf16_np(o_exact - tol), round_bf16_np(o_exact + tol)
    g = g_logits.astype(np.float64)
    bad = np.nonzero(~((g >= lo) & (g <= hi)))[0]
    assert bad.size == 0, (f"{what}: {bad.size} bf16 logits outside the allowed roundings, first "
                           f"token {o_tokens[bad[0]]}: gpu {g[bad[0]]!r} exact {o_exact[bad[0]]!r} "
                           f"oracle {o_logits[bad[0]]!r}")


def check_indices_bf16(o_tokens, o_logits, o_idx, g_logits, g_idx, topk, what=""):
    """bf16 scoring: the GPU's selection is exact for its own bf16 logits (checked by the
    caller); where those equal the oracle's bf16 logits on the whole row, the indices are
    the oracle's exactly (ties included)."""
    if np.array_equal(g_logits.astype(np.float32).view(np.uint32),
                      o_logits.astype(np.float32).view(np.uint32)):
        np.testing.assert_array_equal(g_idx, o_idx, err_msg=f"{what}: indices differ")


class GpuRun:
    """One configured indexer over a device case: schedule + per-layer calls."""

    def __init__(self, case, dcase, sbk=0, q_format="mxfp4", score_format="fp32"):
        import torch

        import sparse_attention_indexer_candidate_amd as idx

        self.idx = idx
        s = case.spec
        self.case, self.dcase, self.spec = case, dcase, s
        self.q_format = q_format
        self.score_format = score_format
        self.cfg = idx.make_config(s.num_heads, s.head_dim,
                                   idx.IDX_Q_MXFP4 if q_format == "mxfp4" else idx.IDX_Q_FP8_E4M3_ROWSCALE,
                                   s.page_size, s.cbs, sbk, s.nb, s.topk,
                                   idx.IDX_SCORE_BF16 if score_format == "bf16" else idx.IDX_SCORE_FP32)
        self.sbk = self.cfg.sparse_block_kv
        R = case.num_rows
        dev = dcase.row_ke.device
        self.rows = idx.make_rows(dcase.row_ke, dcase.row_ks, dcase.row_table, s.next_n)
        self.sched = idx.Schedule(self.cfg, R, dev)
        self.kcaches = [idx.make_kcache(L.pool, s.page_size, s.head_dim, dcase.block_table)
                        for L in dcase.layers]
        self.out = torch.full((R, s.topk), -7, dtype=torch.int32, device=dev)
        self.logits = torch.empty((R, s.nb * s.cbs), dtype=torch.float32, device=dev)
        ws = idx.idx_workspace_bytes(self.cfg, R, 0)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)

    def expand(self, layer=0):
        self.idx.idx_expand_candidates(self.cfg, self.rows, self.kcaches[layer],
                                       self.dcase.candidate_blocks,
                                       self.dcase.candidate_blocks.stride(0), self.sched.struct)

    def score(self, layer=0, with_logits=True):
        L = self.dcase.layers[layer]
        qv, qs = L.q(self.q_format)
        self.idx.idx_sparse_mqa_logits_topk(
            self.cfg, self.rows, qv, qs, L.w(self.score_format), self.kcaches[layer], self.sched.struct,
            self.out, self.out.stride(0), self.logits if with_logits else None,
            None if with_logits else self.workspace,
            0 if with_logits else self.workspace.numel())

    def score_layers(self, layers, with_logits, workspace_layers=1, out_pad=0,
                     expand_in_call=False):
        """One idx_sparse_mqa_logits_topk_layers call over the given layers; returns
        per-layer (indices, logits or None) device tensors.  with_logits[i] False: that
        layer writes no logits (the workspace serves it).  workspace_layers: the
        workspace holds that many layers' logits (all of them lets fewer rows than CUs
        run every layer in one split launch).  out_pad: each layer's indices are a view
        of a [rows][topk + out_pad] buffer filled with -7 (out_stride topk + out_pad),
        whose extra columns padded_tail reads.  expand_in_call: one
        idx_expand_and_score_layers call instead, which also builds the schedule."""
        import torch

        R, s = self.case.num_rows, self.spec
        dev = self.dcase.row_ke.device
        outs, logs, entries = [], [], []
        for layer, wl in zip(layers, with_logits):
            L = self.dcase.layers[layer]
            qv, qs = L.q(self.q_format)
            out = torch.full((R, s.topk + out_pad), -7, dtype=torch.int32, device=dev)
            out = out[:, :s.topk]
            lg = torch.empty((R, s.nb * s.cbs), dtype=torch.float32, device=dev) if wl else None
            outs.append(out)
            logs.append(lg)
            entries.append((qv, qs, L.w(self.score_format), self.kcaches[layer], out, lg))
        ws = self.workspace
        if workspace_layers > 1:
            ws = torch.empty(self.idx.idx_workspace_bytes(self.cfg, R * workspace_layers, 0),
                             dtype=torch.uint8, device=dev)
        if expand_in_call:
            cand = self.dcase.candidate_blocks
            self.idx.idx_expand_and_score_layers(self.cfg, self.rows, cand, cand.stride(0),
                                                 self.sched.struct, entries, s.topk + out_pad,
                                                 ws, ws.numel())
        else:
            self.idx.idx_sparse_mqa_logits_topk_layers(self.cfg, self.rows, self.sched.struct,
                                                       entries, s.topk + out_pad, ws, ws.numel())
        return outs, logs


    def fetch(self):
        import torch

        torch.cuda.synchronize()
        return dict(indices=self.out.cpu().numpy(), logits=self.logits.cpu().numpy(),
                    sparse_indices=self.sched.sparse_indices.cpu().numpy(),
                    end=self.sched.end.cpu().numpy(),
                    kept=self.sched.work[:4 * self.case.num_rows].view(torch.int32).cpu().numpy())


def padded_tail(out_view, pad):
    """The pad columns [topk, topk + pad) of a score_layers output view, on the host."""
    import torch

    R, k = out_view.shape
    full = torch.as_strided(out_view, (R, k + pad), (out_view.stride(0), 1))
    return full[:, k:].cpu().numpy()

def compare_rows(case, res, ora, topk, sbk, what="", ora_scale=None, score_format="fp32"):
    """Compare GPU results (dict from GpuRun.fetch) with an oracle RowResult; ora_scale
    (optional) is the oracle's RowResult for the same rows with |w| (see check_logits).
    score_format "bf16": the bf16 rules above (ora from the oracle's bf16 scoring)."""
    for i, r in enumerate(ora.rows):
        r = int(r)
        tag = f"{what} row {r}"
        ks, ke = int(case.row_ks[r]), int(case.row_ke[r])
        gt, gl = gpu_row_tokens(res["sparse_indices"][r], int(res["kept"][r]), sbk, ks, ke,
                                res["logits"][r])
        assert res["end"][r] == ora.count[i], f"{tag}: end {res['end'][r]} != {ora.count[i]}"
        if score_format == "bf16":
            check_logits_bf16(ora.row_tokens(i), ora.row_exact(i), ora.row_logits(i), gt, gl, tag)
            check_topk_exact_for_own_logits(gt, gl, res["indices"][r], topk, tag)
            check_indices_bf16(ora.row_tokens(i), ora.row_logits(i), ora.indices[i], gl,
                               res["indices"][r], topk, tag)
            continue
        sc = None if ora_scale is None else ora_scale.row_logits(i)
        check_logits(ora.row_tokens(i), ora.row_logits(i), gt, gl, tag, sc)
        check_indices(ora.row_tokens(i), ora.row_logits(i), ora.indices[i], res["indices"][r],
                      topk, tag, sc)
        check_topk_exact_for_own_logits(gt, gl, res["indices"][r], topk, tag)


def corrupt_tables(case, seed):
    """Inputs that break the K cache's preconditions, and the inputs the oracle scores in
    their place.

    Returns (bad, clean, bad_rows, bad_pages).  bad: about an eighth of the block-table
    entries that in-range candidates reach point outside the pool (-1, num_pages + 3 and
    INT32_MAX in turn), and two rows' table rows lie outside [0, num_tables) (-1 and
    num_tables).  The library drops the sparse blocks of such pages and rows from the
    schedule without reading them, so its result on bad is the oracle's on clean: the
    original tables, with every candidate block on a corrupted page removed (-1) and no
    candidates for the two rows.  Requires cbs <= page_size (a candidate block lies in one
    page).  bad_pages: bool [num_tables, pages_per_table], True where an entry was
    corrupted."""
    import workloads as W

    s = case.spec
    assert s.cbs <= s.page_size and s.page_size % s.cbs == 0, "a candidate block in one page"
    rng = np.random.default_rng(seed)
    T, P = case.block_table.shape
    cand = case.candidate_blocks
    reach = np.zeros((T, P), bool)
    for r in range(case.num_rows):
        c = cand[r]
        c = c[(c >= 0) & (c.astype(np.int64) * s.cbs < case.row_ke[r])]
        lp = c.astype(np.int64) * s.cbs // s.page_size
        reach[case.row_table[r], lp[lp < P]] = True
    ti, pi = np.nonzero(reach & (case.block_table >= 0))
    pick = rng.choice(len(ti), size=max(3, len(ti) // 8), replace=False)
    bad_bt = case.block_table.copy()
    num_pages = case.layers[0].num_pages
    outside = np.array([-1, num_pages + 3, np.iinfo(np.int32).max], np.int64)
    bad_bt[ti[pick], pi[pick]] = outside[np.arange(len(pick)) % 3]
    bad_pages = np.zeros((T, P), bool)
    bad_pages[ti[pick], pi[pick]] = True
    bad_rows = rng.choice(case.num_rows, size=2, replace=False)
    bad_rt = case.row_table.copy()
    bad_rt[bad_rows[0]] = -1
    bad_rt[bad_rows[1]] = T
    clean = cand.copy()
    for r in range(case.num_rows):
        lp = np.maximum(clean[r].astype(np.int64), 0) * s.cbs // s.page_size
        hit = (clean[r] >= 0) & (lp < P) & bad_pages[case.row_table[r], np.minimum(lp, P - 1)]
        clean[r, hit] = -1
    clean[bad_rows] = -1
    bad = W.Case(s, case.seed, case.row_ks, case.row_ke, bad_rt.astype(np.int32),
                 bad_bt.astype(np.int32), cand, case.layers)
    good = W.Case(s, case.seed, case.row_ks, case.row_ke, case.row_table, case.block_table,
                  clean.astype(np.int32), case.layers)
    return bad, good, bad_rows, bad_pages
