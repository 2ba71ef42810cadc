"""Dense-logits-then-mask brute force, the independent check of the oracle.

Written separately from oracle/oracle.c and structured differently: it builds the
whole dense K matrix of a row by walking its block table, scores *every* position
of [0, ke) with numpy, then masks to the candidate blocks and [ks, ke) and sorts
everything.  The sparse indexer replaces exactly this computation (dense logits
over the context, then a candidate mask: module summary of the vLLM
sparse_mqa_indexer page), so the two must agree.

Element decodes come from outside the oracle: e2m1 from the hand-derived table in
tests/golden/e2m1_codes.txt, UE8M0 and e4m3fn from PyTorch's float8_e8m0fnu and
float8_e4m3fn conversions.  Tiny inputs only.
"""
import math
from fractions import Fraction

import numpy as np
import torch

from golden_io import e2m1_table

_E2M1 = np.array([e2m1_table()[c] for c in range(16)], dtype=np.float64)
_UE8M0 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
_E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] values (low nibble first)."""
    lo = _E2M1[packed & 15]
    hi = _E2M1[packed >> 4]
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dense_k(case, layer, table_row, n_tokens, pool):
    s = case.spec
    D, ps, vb = s.head_dim, s.page_size, s.values_bytes
    K = np.zeros((n_tokens, D))
    for t in range(n_tokens):
        page = table_row[t // ps]
        j = t % ps
        vals = pool[page, j * (D // 2):(j + 1) * (D // 2)]
        sc = pool[page, vb + j * (D // 32): vb + (j + 1) * (D // 32)]
        K[t] = unpack_e2m1(vals) * np.repeat(_UE8M0[sc], 32)
    return K


def q_matrix(case, layer, r, q_format):
    s = case.spec
    L = case.layers[layer]
    if q_format == "mxfp4":
        return unpack_e2m1(L.q_values[r]) * np.repeat(_UE8M0[L.q_scales[r]], 32, axis=-1), 1.0
    return _E4M3[L.q_fp8[r]], float(L.q_rowscale[r])


def round_bf16_exact(x: float) -> float:
    """x rounded to the nearest bf16 value in exact rational arithmetic: the two bf16
    neighbours of |x| at the binade's spacing, the nearer one, a tie to the one with an
    even significand; at or past 2^128 infinity."""
    if x == 0.0 or not math.isfinite(x):
        return x
    a = Fraction(abs(x))
    e = 0
    while Fraction(2) ** e <= a:
        e += 1
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    spacing = Fraction(2) ** max(e - 8, -133)
    lo = (a // spacing) * spacing
    hi = lo + spacing
    if a - lo < hi - a:
        v = lo
    elif hi - a < a - lo:
        v = hi
    else:
        v = lo if (lo / spacing) % 2 == 0 else hi
    v = math.inf if v >= Fraction(2) ** 128 else float(v)
    return -v if x < 0 else v


def weights(L, r, score_format):
    """Row r's head weights as fp64: fp32, or the bf16 codes decoded by PyTorch."""
    if score_format == "bf16":
        codes = torch.from_numpy(L.weights_bf16[r].view(np.int16).copy())
        return codes.view(torch.bfloat16).to(torch.float64).numpy()
    return L.weights[r].astype(np.float64)


def dense_logits(case, r, layer=0, q_format="mxfp4", pool=None, score_format="fp32"):
    """The logits of every position t < ke of row r (fp32, or bf16-rounded held in fp32)."""
    s = case.spec
    L = case.layers[layer]
    if pool is None:
        pool = L.host_pool(s.page_bytes)
    ke = int(case.row_ke[r])
    table_row = case.block_table[case.row_table[r]]
    K = dense_k(case, layer, table_row, ke, pool)
    Q, rs = q_matrix(case, layer, r, q_format)
    S = Q @ K.T                                  # [H, ke], exact in fp64 for these inputs
    if q_format == "fp8":
        S = S * rs
    relu = np.where(S > 0, S, 0.0)                  # ReLU(NaN) = 0
    w = weights(L, r, score_format)
    acc = np.zeros(ke)
    for h in range(s.num_heads):                 # head sum in index order
        acc = acc + w[h] * relu[h]
    acc = np.where(np.isnan(acc), -np.inf, acc)     # a NaN logit ranks as -inf
    if score_format == "bf16":
        return np.array([round_bf16_exact(float(v)) for v in acc], dtype=np.float32)
    return acc.astype(np.float32)


def row(case, r, layer=0, q_format="mxfp4", pool=None, score_format="fp32"):
    """(indices[topk], candidate tokens, their logits) for row r (fp32 logits, or
    bf16-rounded ones held in fp32 with score_format "bf16")."""
    s = case.spec
    ks, ke = int(case.row_ks[r]), int(case.row_ke[r])
    logits = dense_logits(case, r, layer, q_format, pool, score_format)
    blocks = set(int(b) for b in case.candidate_blocks[r] if b >= 0)
    t = np.arange(ke)
    keep = (t >= ks) & np.isin(t // s.cbs, np.array(sorted(blocks), dtype=np.int64))
    tk, lk = t[keep], logits[keep]
    order = np.lexsort((tk, -lk.astype(np.float64)))
    count = min(s.topk, tk.size)
    out = np.full(s.topk, -1, dtype=np.int32)
    out[:count] = np.sort(tk[order[:count]])
    return out, tk.astype(np.int32), lk


def source_row(case, r, nb, layer=0, q_format="mxfp4", pool=None, score_format="fp32"):
    """The candidate-source publication of row r: every position's logit, block maxima
    over [ks, ke) with numpy's maximum.reduceat, the nb best blocks by a full lexsort
    (score descending, block ascending), ascending, -1 padded.  Returns (blocks[nb],
    {block: score})."""
    s = case.spec
    ks, ke = int(case.row_ks[r]), int(case.row_ke[r])
    logits = dense_logits(case, r, layer, q_format, pool, score_format)
    first, last = ks // s.cbs, (ke - 1) // s.cbs if ke > ks else -1
    ids = np.arange(first, last + 1)
    scores = {}
    if ids.size:
        starts = np.maximum(ids * s.cbs, ks) - ks
        m = np.maximum.reduceat(logits[ks:ke], starts)
        scores = {int(b): float(v) for b, v in zip(ids, m)}
    b = np.array(sorted(scores), dtype=np.int64)
    v = np.array([scores[int(x)] for x in b], dtype=np.float64)
    order = np.lexsort((b, -v)) if b.size else np.zeros(0, np.int64)
    count = min(nb, b.size)
    out = np.full(nb, -1, np.int32)
    out[:count] = np.sort(b[order[:count]])
    return out, scores
