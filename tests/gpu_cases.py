"""Shared pieces of the GPU parity tests: the runner that calls the HIP path through the C
ABI and compares it with the oracle on every row, case tables several test files use, and
input rewriters (signed or zero weights, overflowing or NaN inputs).  Not a test file."""

import numpy as np
import torch

import oracle
import workloads as W
from parity import GpuRun, compare_rows, padded_tail
from workloads.device import to_device


DEV = "cuda:0"


THREADS = oracle.default_threads()


def _say(msg):
    print(msg, flush=True)


def run_and_compare(case, rows=None, layers=(0,), q_format="mxfp4", sbk=0, tag="", scale_case=None,
                    score_format="fp32"):
    dcase = to_device(case, DEV)
    g = GpuRun(case, dcase, sbk=sbk, q_format=q_format, score_format=score_format)
    _say(f"[{tag}] expand rows={case.num_rows} sbk={g.sbk} fmt={q_format}")
    g.expand()
    si_o, end_o = oracle.expand(case, g.sbk)
    res = None
    for layer in layers:
        _say(f"[{tag}] score layer {layer}")
        g.score(layer, with_logits=True)
        res = g.fetch()
        np.testing.assert_array_equal(res["sparse_indices"], si_o, err_msg=f"{tag}: schedule")
        np.testing.assert_array_equal(res["end"], end_o, err_msg=f"{tag}: end")
        pool = case.layers[layer].host_pool(case.spec.page_bytes)
        ora = oracle.indexer_rows(case, layer, rows, q_format, pool=pool, threads=THREADS,
                                  score_format=score_format)
        ora_scale = None
        if scale_case is not None:   # same inputs with |w|: the tolerance's magnitudes
            ora_scale = oracle.indexer_rows(scale_case, layer, rows, q_format, pool=pool,
                                            threads=THREADS)
        compare_rows(case, res, ora, case.spec.topk, g.sbk, f"{tag} layer {layer}", ora_scale,
                     score_format=score_format)
        # the launch configuration of the benchmark (workspace, no logits output)
        g.out.fill_(-7)
        g.score(layer, with_logits=False)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(g.out.cpu().numpy(), res["indices"],
                                      err_msg=f"{tag}: workspace launch differs")
    return g, res


SMALL = {
    "ragged_sbk64_ks": W.Spec(name="s1", num_rows=37, num_heads=64, head_dim=128, page_size=128,
                              cbs=128, nb=7, topk=100, ke_rule="uniform", ke_lo=1, ke_hi=3000,
                              ks_rule="random", cand_rule="messy", fill="all"),
    "sbk16": W.Spec(name="s2", num_rows=20, page_size=32, cbs=16, nb=40, topk=50,
                    ke_rule="uniform", ke_lo=100, ke_hi=900, cand_rule="messy", fill="all"),
    "sbk32_k_above_valid": W.Spec(name="s3", num_rows=13, page_size=64, cbs=32, nb=20, topk=300,
                                  ke_rule="uniform", ke_lo=50, ke_hi=1500, ks_rule="random",
                                  cand_rule="distinct", fill="all"),
    "prefill_offset": W.Spec(name="s4", num_rows=300, page_size=64, cbs=64, nb=16, topk=128,
                             mode="prefill", ke_rule="causal", row_offset=100, context=512,
                             cand_rule="causal_all", fill="all"),
    "empty_and_tiny_rows": W.Spec(name="s5", num_rows=9, page_size=64, cbs=64, nb=4, topk=64,
                                  ke_rule="uniform", ke_lo=0, ke_hi=70, cand_rule="distinct",
                                  fill="all"),
    "cbs128_split_sbk32": W.Spec(name="s6", num_rows=11, page_size=128, cbs=128, nb=9, topk=200,
                                 ke_rule="uniform", ke_lo=300, ke_hi=2000, ks_rule="random",
                                 cand_rule="messy", fill="all"),
    # >= 2 rows per CU, MXFP4: the one-row kernel with two 8-wave rows a CU
    "two_rows_a_cu": W.Spec(name="s12", num_rows=600, page_size=64, cbs=64, nb=20, topk=200,
                            ke_rule="uniform", ke_lo=1, ke_hi=2500, ks_rule="random",
                            cand_rule="messy", fill="all"),
    "two_rows_a_cu_sbk16": W.Spec(name="s13", num_rows=520, page_size=32, cbs=16, nb=60, topk=90,
                                  ke_rule="uniform", ke_lo=50, ke_hi=1200, cand_rule="messy",
                                  fill="all"),
    # >= 8 rows per CU: the row-group kernel (2 rows per workgroup); rows on one table
    # share K tiles, a ragged last group, messy candidates and ks > 0
    "rowgroup_shared_table_messy": W.Spec(name="s7", num_rows=2051, page_size=128, cbs=64, nb=8,
                                          topk=100, mode="prefill", ke_rule="uniform", ke_lo=1,
                                          ke_hi=1500, ks_rule="random", context=1600,
                                          cand_rule="messy", fill="all"),
    # ... and rows on their own table rows (no sharing), k above the valid count
    "rowgroup_own_tables": W.Spec(name="s8", num_rows=2048, page_size=64, cbs=64, nb=6, topk=300,
                                  ke_rule="uniform", ke_lo=10, ke_hi=3000,
                                  cand_rule="distinct", fill="all"),
    # a prefill chunk's K packed into one page holding every position (the contiguous
    # K-workspace form of the prefill path): one block-table entry, on the split,
    # one-row-per-workgroup and row-group kernels
    "one_page_workspace_split": W.Spec(name="s9", num_rows=40, page_size=2048, cbs=64, nb=16,
                                       topk=128, mode="prefill", ke_rule="uniform", ke_lo=1,
                                       ke_hi=2048, ks_rule="random", context=2048,
                                       cand_rule="messy", fill="all"),
    "one_page_workspace_rows": W.Spec(name="s10", num_rows=300, page_size=2048, cbs=64, nb=16,
                                      topk=128, mode="prefill", ke_rule="uniform", ke_lo=1,
                                      ke_hi=2048, ks_rule="random", context=2048,
                                      cand_rule="messy", fill="all"),
    "one_page_workspace_rowgroups": W.Spec(name="s11", num_rows=2050, page_size=2048, cbs=64,
                                           nb=8, topk=100, mode="prefill", ke_rule="uniform",
                                           ke_lo=1, ke_hi=2048, ks_rule="random", context=2048,
                                           cand_rule="messy", fill="all"),
    # top-1 (a single survivor of the radix search) on the split, one-row and row-group kernels
    "topk1_split": W.Spec(name="s14", num_rows=30, page_size=64, cbs=64, nb=10, topk=1,
                          ke_rule="uniform", ke_lo=1, ke_hi=2000, ks_rule="random",
                          cand_rule="messy", fill="all"),
    "topk1_rows": W.Spec(name="s15", num_rows=300, page_size=64, cbs=64, nb=10, topk=1,
                         ke_rule="uniform", ke_lo=1, ke_hi=2000, ks_rule="random",
                         cand_rule="messy", fill="all"),
    "topk1_rowgroups": W.Spec(name="s16", num_rows=2050, page_size=64, cbs=64, nb=8, topk=1,
                              mode="prefill", ke_rule="uniform", ke_lo=1, ke_hi=1500,
                              ks_rule="random", context=1600, cand_rule="messy", fill="all"),
    # the expansion's register sort at each width: 2 ids a lane just past 128 candidates is
    # the smallest 4-id case, 256 the largest; 512 (16-token blocks, 8192 columns) the
    # 8-id maximum; and 4 ids a lane on the one-row kernel
    "nb129_e4": W.Spec(name="s18", num_rows=24, page_size=32, cbs=32, nb=129, topk=1000,
                       ke_rule="uniform", ke_lo=1000, ke_hi=9000, ks_rule="random",
                       cand_rule="messy", fill="all"),
    "nb256_e4": W.Spec(name="s19", num_rows=20, page_size=16, cbs=16, nb=256, topk=2000,
                       ke_rule="uniform", ke_lo=500, ke_hi=9000, ks_rule="random",
                       cand_rule="messy", fill="all"),
    "nb512_e8": W.Spec(name="s20", num_rows=16, page_size=16, cbs=16, nb=512, topk=4000,
                       ke_rule="uniform", ke_lo=2000, ke_hi=12000, ks_rule="random",
                       cand_rule="messy", fill="all"),
    "nb200_e4_rows": W.Spec(name="s21", num_rows=300, page_size=32, cbs=32, nb=200, topk=1500,
                            ke_rule="uniform", ke_lo=1000, ke_hi=9000, cand_rule="messy",
                            fill="all"),
    # candidate blocks of four pages each (cbs 256 on 64-token pages: four sparse blocks a
    # candidate, each on its own page)
    "cbs256_pages64": W.Spec(name="s17", num_rows=25, page_size=64, cbs=256, nb=6, topk=200,
                             ke_rule="uniform", ke_lo=100, ke_hi=3000, ks_rule="random",
                             cand_rule="messy", fill="all"),
}


def _random_spec(i):
    """A seeded random shape for the kernel path i % 3 (split, one row per workgroup,
    row groups): block and page sizes, k, ranges, candidate mess and weight sign vary."""
    rng = np.random.default_rng(1000 + i)
    path = i % 3
    cbs = int(rng.choice([16, 32, 64, 128] if path != 2 else [64, 128]))
    sbk = 64 if cbs % 64 == 0 else cbs
    page_size = int(rng.choice([p for p in (16, 32, 64, 128) if p % sbk == 0]))
    nb = int(rng.integers(1, max(2, min(24, 3000 // cbs))))
    topk = int(rng.integers(1, nb * cbs + 1))
    rows = [int(rng.integers(1, 200)), int(rng.integers(256, 360)), 2048 + int(rng.integers(0, 40))][path]
    ke_hi = int(rng.integers(64, 5000))
    common = dict(name=f"rand{i}", num_rows=rows, page_size=page_size, cbs=cbs, nb=nb, topk=topk,
                  ks_rule=str(rng.choice(["zero", "random"])), fill="all",
                  cand_rule=str(rng.choice(["messy", "distinct"])))
    if path == 2:   # rows on one table (a prefill chunk's shape)
        return W.Spec(mode="prefill", ke_rule="uniform", ke_lo=1, ke_hi=ke_hi, context=ke_hi,
                      **common), bool(rng.random() < 0.5)
    return W.Spec(ke_rule="uniform", ke_lo=int(rng.integers(0, ke_hi)), ke_hi=ke_hi,
                  **common), bool(rng.random() < 0.5)


def _reweighted(case, kind, seed):
    """The case with every layer's head weights replaced.  "signed": U(-1, 1) / 8, so
    logits take both signs (the negative half of the key order and of the first radix
    digit); "zero": every logit is +0, one tie across the whole row that only the
    lower-token rule decides."""
    import dataclasses

    rng = np.random.default_rng(seed)
    layers = []
    for L in case.layers:
        if kind == "signed":
            w = ((rng.random(L.weights.shape) * 2.0 - 1.0) / 8.0).astype(np.float32)
        else:
            w = np.zeros_like(L.weights)
        layers.append(dataclasses.replace(L, weights=w))
    return dataclasses.replace(case, layers=layers)


def _dense_indices(g, case, ctx):
    import sparse_attention_indexer_candidate_amd as idx

    R = case.num_rows
    dout = torch.full((R, case.spec.topk), -7, dtype=torch.int32, device=DEV)
    dlog = torch.empty((R, ctx), dtype=torch.float32, device=DEV)
    L = g.dcase.layers[0]
    qv, qs = L.q("mxfp4")
    idx.idx_dense_masked_logits_topk(g.cfg, g.rows, ctx, qv, qs, L.weights, g.kcaches[0],
                                     g.sched.struct, dout, dout.stride(0), dlog, dlog.stride(0))
    torch.cuda.synchronize()
    return dout.cpu().numpy()


# one case per scoring/selection kernel: fewer rows than CUs (split scoring, separate
# selection), at least one row per CU (one workgroup a row), 8+ rows per CU on one
# table (row groups)
WEIGHT_PATHS = {
    "split": SMALL["ragged_sbk64_ks"],
    "fused": W.Spec(name="wf", num_rows=300, page_size=64, cbs=64, nb=8, topk=200,
                    ke_rule="uniform", ke_lo=10, ke_hi=1500, ks_rule="random",
                    cand_rule="messy", fill="all"),
    "rowgroup": SMALL["rowgroup_shared_table_messy"],
}


def _overflowed(case, frac, seed):
    """The case with a fraction of its K tokens made to overflow: every query head's
    first 32-element block is 1.0 at scale 2^13 (the other blocks keep their codes at
    that scale), the chosen tokens' first block is 6.0 at scale 2^127, and every head
    weight is negative, so those tokens' logits are -inf in fp32 (GPU accumulation and
    the oracle's fp64 sum rounded to fp32 alike) while the other logits stay finite."""
    import dataclasses

    s = case.spec
    rng = np.random.default_rng(seed)
    vb = s.values_bytes
    layers = []
    for L in case.layers:
        qv = L.q_values.copy()
        qv[:, :, :16] = 0x22                      # e2m1 1.0 in both nibbles
        qs = np.full_like(L.q_scales, 127 + 13)
        data = L.filled_data.copy()
        hit = rng.random((data.shape[0], s.page_size)) < frac
        for p, slot in zip(*np.nonzero(hit)):
            data[p, slot * (s.head_dim // 2):slot * (s.head_dim // 2) + 16] = 0x77   # 6.0
            data[p, vb + slot * (s.head_dim // 32)] = 254                          # 2^127
        w = -(rng.random(L.weights.shape) / 8.0 + 1e-3).astype(np.float32)
        layers.append(dataclasses.replace(L, q_values=qv, q_scales=qs, filled_data=data,
                                          weights=w))
    return dataclasses.replace(case, layers=layers)


# Block-table entries outside the pool and table rows outside [0, num_tables), on each
# launch shape: split rows, one row per workgroup (128-token pages, two candidate blocks
# a page), row groups (a prefill chunk on one table)
DROPPED = {
    "split": W.Spec(name="dr1", num_rows=40, page_size=64, cbs=64, nb=16, topk=200,
                    ke_rule="uniform", ke_lo=300, ke_hi=3000, ks_rule="random",
                    cand_rule="messy", fill="all"),
    "one_row": W.Spec(name="dr2", num_rows=300, page_size=128, cbs=64, nb=20, topk=150,
                      ke_rule="uniform", ke_lo=300, ke_hi=3000, ks_rule="random",
                      cand_rule="messy", fill="all"),
    "row_groups": W.Spec(name="dr3", num_rows=2050, page_size=64, cbs=64, nb=8, topk=100,
                         mode="prefill", ke_rule="uniform", ke_lo=1, ke_hi=1500,
                         ks_rule="random", context=1600, cand_rule="messy", fill="all"),
}


def _sweep_spec(name, rows, cbs, nb, layers=1, prefill=False, topk=None):
    """A small case for one launch form: cbs sets the sparse block (64 for cbs 64, else
    cbs) and nb the row width (nb * cbs columns)."""
    common = dict(name=name, num_rows=rows, page_size=max(cbs, 32) if cbs < 64 else 64, cbs=cbs,
                  nb=nb, topk=topk or min(500, nb * cbs), layers=layers,
                  q_formats=("mxfp4", "fp8"), fill="all")
    if prefill:
        return W.Spec(mode="prefill", ke_rule="uniform", ke_lo=1, ke_hi=nb * cbs,
                      context=nb * cbs, ks_rule="random", cand_rule="messy", **common)
    return W.Spec(ke_rule="uniform", ke_lo=nb * cbs // 2, ke_hi=2 * nb * cbs, ks_rule="random",
                  cand_rule="messy", **common)


def _check_layers_call(case, name, q_format, score_format="fp32"):
    """One multi-layer call (and its full-workspace and all-logits forms) against one call
    per layer, bit for bit, and every layer against the oracle on every row."""
    nl = case.spec.layers
    g = GpuRun(case, to_device(case, DEV), q_format=q_format, score_format=score_format)
    g.expand()
    with_logits = [i % 2 == 0 for i in range(nl)]     # odd layers use the workspace
    _say(f"[layers-{name}-{q_format}] one call, {nl} layers")
    outs, logs = g.score_layers(range(nl), with_logits)
    torch.cuda.synchronize()
    # a workspace for every layer's logits, and every layer with its own logits: fewer rows
    # than CUs then take the batched split launches
    _say(f"[layers-{name}-{q_format}] workspace for all layers")
    outs_w, logs_w = g.score_layers(range(nl), with_logits, workspace_layers=nl)
    _say(f"[layers-{name}-{q_format}] every layer with logits")
    outs_a, logs_a = g.score_layers(range(nl), [True] * nl)
    _say(f"[layers-{name}-{q_format}] output rows wider than k")
    outs_p, _ = g.score_layers(range(nl), with_logits, out_pad=5)
    torch.cuda.synchronize()
    for layer in range(nl):
        np.testing.assert_array_equal(outs_p[layer].cpu().numpy(), outs[layer].cpu().numpy(),
                                      err_msg=f"{name} layer {layer}: out_stride k + 5")
        assert np.all(padded_tail(outs_p[layer], 5) == -7), f"{name} layer {layer}: wrote past k"
    for layer in range(nl):
        np.testing.assert_array_equal(outs_w[layer].cpu().numpy(), outs[layer].cpu().numpy(),
                                      err_msg=f"{name} layer {layer}: full workspace")
        np.testing.assert_array_equal(outs_a[layer].cpu().numpy(), outs[layer].cpu().numpy(),
                                      err_msg=f"{name} layer {layer}: all logits")
        np.testing.assert_array_equal(logs_a[layer].cpu().numpy().view(np.uint32),
                                      (logs[layer] if logs[layer] is not None else logs_a[layer])
                                      .cpu().numpy().view(np.uint32))
    for layer in range(nl):
        _say(f"[layers-{name}-{q_format}] layer {layer} against its own call")
        g.out.fill_(-7)
        g.score(layer, with_logits=True)
        res = g.fetch()
        np.testing.assert_array_equal(outs[layer].cpu().numpy(), res["indices"],
                                      err_msg=f"{name} layer {layer}: indices")
        if logs[layer] is not None:
            np.testing.assert_array_equal(logs[layer].cpu().numpy().view(np.uint32),
                                          res["logits"].view(np.uint32),
                                          err_msg=f"{name} layer {layer}: logits")
        pool = case.layers[layer].host_pool(case.spec.page_bytes)
        ora = oracle.indexer_rows(case, layer, None, q_format, pool=pool, threads=THREADS,
                                  score_format=score_format)
        res["indices"] = outs[layer].cpu().numpy()
        compare_rows(case, res, ora, case.spec.topk, g.sbk, f"layers-{name} layer {layer}",
                     score_format=score_format)


# ---------------------------------------------------------------- NaN inputs ------
# One rule on both sides: a NaN scale byte (UE8M0 0xFF) or e4m3 code makes a NaN dot
# product, which ReLU maps to 0 (the matrix cores return NaN with the sign bit set, and
# the kernels' ReLU is an integer max); a NaN logit (a NaN weight) ranks as -inf (lowest,
# ties toward the lower token), so the selection's counts and keys always agree.

def _with_nan_inputs(case, q_format, seed):
    """A copy of the case with K scale byte 0xFF on ~1 % of every row's candidate tokens,
    a NaN query element on one head of row 0 and a NaN weight on row 1."""
    import dataclasses

    rng = np.random.default_rng(seed)
    s = case.spec
    L = case.layers[0]
    data = L.filled_data.copy()
    for r in range(case.num_rows):
        toks = oracle.candidate_tokens(case.candidate_blocks[r], s.cbs, int(case.row_ks[r]),
                                       int(case.row_ke[r]))
        for t in rng.choice(toks, size=max(1, toks.size // 100), replace=False) if toks.size else []:
            page = case.block_table[case.row_table[r], t // s.page_size]
            i = int(np.searchsorted(L.filled_pages, page))
            data[i, s.values_bytes + (t % s.page_size) * (s.head_dim // 32) + int(rng.integers(4))] = 0xFF
    w = L.weights.copy()
    w[1, 33] = np.nan
    kw = dict(filled_data=data, weights=w)
    if q_format == "mxfp4":
        qs = L.q_scales.copy()
        qs[0, 7, 1] = 0xFF
        kw["q_scales"] = qs
    else:
        q8 = L.q_fp8.copy()
        q8[0, 7, 40] = 0x7F          # e4m3fn S.1111.111: NaN
        kw["q_fp8"] = q8
    return dataclasses.replace(case, layers=[dataclasses.replace(L, **kw)] + case.layers[1:])
