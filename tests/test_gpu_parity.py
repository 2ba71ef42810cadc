"""GPU parity of the HIP path against the CPU oracle, called through the C ABI.

Small cases span several 64-column groups, ragged tails, every sparse block size,
ks > 0, duplicate / -1 / out-of-range candidates, empty rows and k above and below
the valid count; they are compared on every row.  The five workloads run at their
full sizes in the launch configuration the benchmark uses and are compared with the
oracle on every row (the oracle runs the rows on all host cores at once), plus
properties checked on every row at any size.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import GpuRun, compare_rows, corrupt_tables, exact_topk, gpu_row_tokens, padded_tail
from workloads.device import to_device

pytestmark = pytest.mark.gpu
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


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_cases_all_rows(name):
    spec = SMALL[name]
    sbk = 32 if name == "cbs128_split_sbk32" else 0
    run_and_compare(W.generate(spec, seed=11), sbk=sbk, tag=name)


def test_small_case_fp8_query():
    spec = W.Spec(name="f8", num_rows=21, page_size=64, cbs=64, nb=12, topk=150,
                  ke_rule="uniform", ke_lo=10, ke_hi=2500, ks_rule="random", cand_rule="messy",
                  fill="all", q_formats=("mxfp4", "fp8"))
    case = W.generate(spec, seed=5)
    run_and_compare(case, q_format="fp8", tag="fp8")


def test_fp8_query_rows_per_cu():
    """fp8 queries with at least as many rows as CUs: the one-row-per-workgroup kernel."""
    spec = W.Spec(name="f8r", num_rows=300, page_size=64, cbs=64, nb=8, topk=200,
                  ke_rule="uniform", ke_lo=10, ke_hi=1500, ks_rule="random", cand_rule="messy",
                  fill="all", q_formats=("mxfp4", "fp8"))
    case = W.generate(spec, seed=7)
    run_and_compare(case, q_format="fp8", tag="fp8_rows")


@pytest.mark.parametrize("shape", ["narrow", "wide", "wide_sbk16"])
def test_fp8_query_two_rows_a_cu(shape):
    """fp8 queries with at least two rows per CU: 4-wave rows, two a CU (32 keys a thread
    at 8192 columns), or 8-wave rows where 16-token sparse blocks are too short for that."""
    specs = {
        "narrow": W.Spec(name="f8n", num_rows=600, page_size=64, cbs=64, nb=12, topk=200,
                         ke_rule="uniform", ke_lo=10, ke_hi=2500, ks_rule="random",
                         cand_rule="messy", fill="all"),
        "wide": W.Spec(name="f8w", num_rows=520, page_size=64, cbs=64, nb=128, topk=2048,
                       ke_rule="uniform", ke_lo=6000, ke_hi=12000, cand_rule="distinct",
                       fill="candidates"),
        "wide_sbk16": W.Spec(name="f8s", num_rows=520, page_size=32, cbs=16, nb=320, topk=1000,
                             ke_rule="uniform", ke_lo=3000, ke_hi=9000, cand_rule="messy",
                             fill="candidates"),
    }
    import dataclasses
    spec = dataclasses.replace(specs[shape], q_formats=("mxfp4", "fp8"))
    run_and_compare(W.generate(spec, seed=11), q_format="fp8", tag=f"fp8_two_rows_{shape}")


def test_row_groups_wide_rows_all_rows():
    """Row groups over more than 4096 candidate columns (the 8192-column workgroup shape):
    2048 prefill rows on one table, 100 candidate blocks of 64, every row against the
    oracle."""
    spec = W.Spec(name="wide", num_rows=2048, page_size=64, cbs=64, nb=100, topk=1500,
                  mode="prefill", ke_rule="uniform", ke_lo=1, ke_hi=7000, ks_rule="random",
                  context=7000, cand_rule="messy", fill="all")
    run_and_compare(W.generate(spec, seed=3), tag="wide")


def test_row_groups_many_short_rows_all_rows():
    """A prefill chunk of 20001 rows (an odd count: the last row group holds one row) of
    short causal rows on one table: 10001 row-group workgroups dispatched heaviest first,
    every row against the oracle."""
    spec = W.Spec(name="many", num_rows=20001, page_size=64, cbs=64, nb=4, topk=100,
                  mode="prefill", ke_rule="uniform", ke_lo=1, ke_hi=256, ks_rule="random",
                  context=256, cand_rule="messy", fill="all")
    import sparse_attention_indexer_candidate_amd as idx

    case = W.generate(spec, seed=11)
    cfg = idx.make_config(page_size=64, candidate_block_size=64, num_candidate_blocks=4, topk=100)
    assert idx.idx_sparse_plan(cfg, case.num_rows, 1)["plan"] == idx.IDX_PLAN_ROW_GROUP
    run_and_compare(case, tag="many")


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


@pytest.mark.parametrize("i", range(20))
def test_random_shapes_all_rows(i):
    import dataclasses

    spec, signed = _random_spec(i)
    case = W.generate(spec, seed=i)
    scale_case = None
    if signed:
        case = _reweighted(case, "signed", seed=i)
        scale_case = dataclasses.replace(
            case, layers=[dataclasses.replace(L, weights=np.abs(L.weights)) for L in case.layers])
    _say(f"[rand{i}] rows={spec.num_rows} cbs={spec.cbs} page={spec.page_size} nb={spec.nb} "
         f"k={spec.topk} ke<={spec.ke_hi} {spec.mode} signed={signed}")
    g, res = run_and_compare(case, tag=f"rand{i}", scale_case=scale_case)
    # the dense comparator on the same inputs: the same logits, so the same indices
    _say(f"[rand{i}] dense")
    ctx = max(64, int(case.row_ke.max() + 63) // 64 * 64)
    np.testing.assert_array_equal(_dense_indices(g, case, ctx), res["indices"],
                                  err_msg=f"rand{i}: dense != sparse indices")


@pytest.mark.parametrize("i", range(12))
def test_random_shapes_fp8_queries_and_bf16_scoring(i):
    """Seeded random shapes (as test_random_shapes_all_rows) with fp8 queries, bf16 scoring
    or both: the split, one-row and many-row launch forms of each (fp8 rows at two or more
    a CU take 4-wave rows; MXFP4 many-row cases take row groups)."""
    import dataclasses

    spec, signed = _random_spec(100 + i)
    q_format = "fp8" if i % 2 == 0 else "mxfp4"
    score_format = "bf16" if i % 4 in (1, 2) else "fp32"
    spec = dataclasses.replace(spec, name=f"rq{i}", q_formats=("mxfp4", "fp8"))
    case = W.generate(spec, seed=50 + i)
    scale_case = None
    if signed and score_format == "fp32":
        case = _reweighted(case, "signed", seed=i)
        scale_case = dataclasses.replace(
            case, layers=[dataclasses.replace(L, weights=np.abs(L.weights)) for L in case.layers])
    _say(f"[rq{i}] rows={spec.num_rows} cbs={spec.cbs} page={spec.page_size} nb={spec.nb} "
         f"k={spec.topk} {spec.mode} {q_format} {score_format} signed={scale_case is not None}")
    run_and_compare(case, tag=f"rq{i}", q_format=q_format, score_format=score_format,
                    scale_case=scale_case)


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


@pytest.mark.parametrize("kind", ["signed", "zero"])
@pytest.mark.parametrize("path", sorted(WEIGHT_PATHS))
def test_signed_and_zero_weights(path, kind):
    import dataclasses

    case = _reweighted(W.generate(WEIGHT_PATHS[path], seed=13), kind, seed=17)
    tag = f"w-{kind}-{path}"
    mag = dataclasses.replace(case, layers=[dataclasses.replace(L, weights=np.abs(L.weights))
                                            for L in case.layers])
    g, res = run_and_compare(case, tag=tag, scale_case=mag)
    k = case.spec.topk
    for i in range(case.num_rows):
        gt, gl = gpu_row_tokens(res["sparse_indices"][i], int(res["kept"][i]), g.sbk,
                                int(case.row_ks[i]), int(case.row_ke[i]), res["logits"][i])
        if kind == "zero":
            assert np.all(gl.view(np.uint32) == 0), f"{tag} row {i}: logits not +0"
            want = np.full(k, -1, np.int32)
            n = min(k, gt.size)
            want[:n] = gt[:n]
            np.testing.assert_array_equal(res["indices"][i], want, err_msg=f"{tag} row {i}")
        else:
            np.testing.assert_array_equal(res["indices"][i], exact_topk(gt, gl, k),
                                          err_msg=f"{tag} row {i}")
    if kind == "signed":
        lg = res["logits"][np.isfinite(res["logits"])]
        assert (lg < 0).any() and (lg > 0).any(), f"{tag}: logits of one sign only"
    if path == "split":
        _say(f"[{tag}] dense")
        ctx = int(case.row_ke.max() + 63) // 64 * 64
        np.testing.assert_array_equal(_dense_indices(g, case, ctx), res["indices"],
                                      err_msg=f"{tag}: dense != sparse indices")


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


@pytest.mark.parametrize("path", sorted(WEIGHT_PATHS))
def test_valid_columns_with_infinite_logits(path):
    """A valid column whose logit overflowed to -inf is still a candidate (the lowest):
    it is selected when k reaches it, exactly as the oracle selects it."""
    case = _overflowed(W.generate(WEIGHT_PATHS[path], seed=13), frac=0.03, seed=19)
    tag = f"inf-{path}"
    g, res = run_and_compare(case, tag=tag)
    ora = oracle.indexer_rows(case, 0, None, "mxfp4",
                              pool=case.layers[0].host_pool(case.spec.page_bytes))
    n_inf = n_chosen = 0
    for i in range(case.num_rows):
        gt, gl = gpu_row_tokens(res["sparse_indices"][i], int(res["kept"][i]), g.sbk,
                                int(case.row_ks[i]), int(case.row_ke[i]), res["logits"][i])
        ol = ora.row_logits(i)
        np.testing.assert_array_equal(np.isneginf(gl), np.isneginf(ol),
                                      err_msg=f"{tag} row {i}: -inf columns differ")
        assert not np.isnan(gl).any(), f"{tag} row {i}: NaN logit"
        np.testing.assert_array_equal(res["indices"][i], ora.indices[i], err_msg=f"{tag} row {i}")
        n_inf += int(np.isneginf(ol).sum())
        n_chosen += int(np.isin(gt[np.isneginf(gl)], res["indices"][i]).sum())
    assert n_inf > 0 and n_chosen > 0, f"{tag}: no -inf column ({n_inf}) or none chosen ({n_chosen})"


# Decode rows in requests of next_n on one table row (MTP / speculative rows) with
# overlapping candidate lists: ragged request counts, ks > 0, 4096- and 8192-column
# shapes, long requests.
MTP = {
    "n2": W.Spec(name="m2", num_rows=40, nb=16, topk=300, ke_rule="uniform", ke_lo=200,
                 ke_hi=3000, cand_rule="mtp_overlap", next_n=2, fill="all"),
    "n3_ks": W.Spec(name="m3", num_rows=33, nb=12, topk=200, ke_rule="uniform", ke_lo=100,
                    ke_hi=2500, ks_rule="random", cand_rule="mtp_overlap", next_n=3,
                    fill="all"),
    "n4_wide": W.Spec(name="m4", num_rows=24, nb=100, topk=1000, ke_rule="uniform",
                      ke_lo=3000, ke_hi=9000, cand_rule="mtp_overlap", next_n=4, fill="all"),
    "n8": W.Spec(name="m8", num_rows=32, nb=20, topk=400, ke_rule="uniform", ke_lo=500,
                 ke_hi=4000, cand_rule="mtp_overlap", next_n=8, mtp_resample=0.5, fill="all"),
}


@pytest.mark.parametrize("name", sorted(MTP))
def test_mtp_decode_rows_share_k(name):
    run_and_compare(W.generate(MTP[name], seed=21), tag=name)


# Enough rows that the placement hint (rows_per_request > 1) permutes whole 64-row blocks:
# the split kernels (130 rows: two blocks and a 2-row tail), one workgroup a row (520 rows)
# and one launch of one-row workgroups for two layers (130 rows x 2).
MTP_PLACED = {
    "n2_split": W.Spec(name="mp2", num_rows=130, nb=16, topk=300, ke_rule="uniform",
                       ke_lo=200, ke_hi=3000, cand_rule="mtp_overlap", next_n=2, fill="all"),
    "n4_one_row": W.Spec(name="mp4", num_rows=520, nb=16, topk=300, ke_rule="uniform",
                         ke_lo=200, ke_hi=3000, cand_rule="mtp_overlap", next_n=4, fill="all"),
    "n2_two_layers": W.Spec(name="mp2l", num_rows=130, nb=16, topk=300, layers=2,
                            ke_rule="uniform", ke_lo=200, ke_hi=3000, cand_rule="mtp_overlap",
                            next_n=2, fill="all"),
}


@pytest.mark.parametrize("name", sorted(MTP_PLACED))
def test_mtp_rows_placed_by_request_match_unplaced_and_oracle(name):
    """The placement hint changes which workgroup scores which row, never a result: every
    row against the oracle, and indices and logits bit for bit against the same calls
    made without the hint."""
    import sparse_attention_indexer_candidate_amd as idx

    case = W.generate(MTP_PLACED[name], seed=23)
    nl = case.spec.layers
    g, _ = run_and_compare(case, layers=tuple(range(nl)), tag=name)
    dcase = g.dcase
    plain = GpuRun(case, dcase)
    plain.rows = idx.make_rows(dcase.row_ke, dcase.row_ks, dcase.row_table, 1)
    plain.expand()
    g.expand()
    for layer in range(nl):
        _say(f"[{name}] layer {layer}: with and without the hint")
        g.score(layer, with_logits=True)
        a = g.fetch()
        plain.score(layer, with_logits=True)
        b = plain.fetch()
        np.testing.assert_array_equal(a["indices"], b["indices"], err_msg=f"{name} {layer}")
        np.testing.assert_array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))
    if nl > 1:
        assert g.idx.idx_sparse_plan(g.cfg, case.num_rows, nl)["plan"] == \
            g.idx.IDX_PLAN_ONE_ROW_LAYERS
        outs, logs = g.score_layers(range(nl), [True] * nl)
        outs_p, logs_p = plain.score_layers(range(nl), [True] * nl)
        torch.cuda.synchronize()
        for layer in range(nl):
            np.testing.assert_array_equal(outs[layer].cpu().numpy(), outs_p[layer].cpu().numpy())
            np.testing.assert_array_equal(logs[layer].cpu().numpy().view(np.uint32),
                                          logs_p[layer].cpu().numpy().view(np.uint32))
            pool = case.layers[layer].host_pool(case.spec.page_bytes)
            ora = oracle.indexer_rows(case, layer, None, "mxfp4", pool=pool, threads=THREADS)
            res = g.fetch()
            res["indices"], res["logits"] = outs[layer].cpu().numpy(), logs[layer].cpu().numpy()
            compare_rows(case, res, ora, case.spec.topk, g.sbk, f"{name} one launch {layer}")


# The kernels' size limits: 8192 candidate columns a row (NB * cbs) and top-k at its
# 8192 maximum (every valid column taken), or 6000 selected of up to 8192.
MAX_WIDTH = {
    "max_width_topk8192_split": W.Spec(name="m1", num_rows=24, page_size=64, cbs=64, nb=128,
                                       topk=8192, ke_rule="uniform", ke_lo=6000, ke_hi=12000,
                                       cand_rule="distinct", fill="candidates"),
    "max_width_select6000_split": W.Spec(name="m2", num_rows=24, page_size=64, cbs=64, nb=128,
                                         topk=6000, ke_rule="uniform", ke_lo=6000, ke_hi=12000,
                                         cand_rule="distinct", fill="candidates"),
}


@pytest.mark.parametrize("name", sorted(MAX_WIDTH))
def test_max_width_split_all_rows(name):
    run_and_compare(W.generate(MAX_WIDTH[name], seed=1), tag=name)


@pytest.mark.parametrize("k,nrows", [(7000, 260), (8192, 260), (8192, 520)])
def test_max_width_rows_per_cu_all_rows(k, nrows):
    """One workgroup a row at the column and top-k limits: 260 rows (one a CU) or 520
    rows (two a CU) of up to 8192 columns, every row against the oracle."""
    spec = W.Spec(name=f"m3_{k}_{nrows}", num_rows=nrows, page_size=64, cbs=64, nb=128,
                  topk=k, ke_rule="uniform", ke_lo=6000, ke_hi=12000, cand_rule="distinct",
                  fill="candidates")
    run_and_compare(W.generate(spec, seed=2), tag=f"maxwidth{k}")


def test_config6_mtp_decode_all_rows():
    run_and_compare(W.generate(W.config(6), 0), tag="cfg6")


def test_config1_tiny_decode_all_rows():
    run_and_compare(W.generate(W.config(1), 0), tag="cfg1")


def test_config2_decode_batch_all_rows():
    run_and_compare(W.generate(W.config(2), 0), tag="cfg2")


def test_config3_prefill_chunk_all_rows():
    case = W.generate(W.config(3), 0)
    g, res = run_and_compare(case, tag="cfg3")
    # rows with i + 1 <= k keep all their tokens 0..i, whatever the arithmetic
    k = case.spec.topk
    for i in range(min(k, case.num_rows)):
        want = np.full(k, -1, np.int32)
        want[:i + 1] = np.arange(i + 1)
        np.testing.assert_array_equal(res["indices"][i], want, err_msg=f"cfg3 row {i}")


def test_config4_long_decode_four_layers_all_rows():
    run_and_compare(W.generate(W.config(4), 0), layers=(0, 1, 2, 3), tag="cfg4")


@pytest.mark.parametrize("q_format", ["mxfp4", "fp8"])
def test_config5_sparse_equals_dense_masked(q_format):
    import sparse_attention_indexer_candidate_amd as idx

    case = W.generate(W.config(5), 0)
    g, res = run_and_compare(case, q_format=q_format, tag=f"cfg5-{q_format}")
    # dense comparator on the same inputs: every token of [0, 65536) scored, masked to
    # the candidates, same selection rule -> identical indices, identical logits
    R, ctx = case.num_rows, 65536
    dlog = torch.empty((R, ctx), dtype=torch.float32, device=DEV)
    dout = torch.full((R, case.spec.topk), -7, dtype=torch.int32, device=DEV)
    L = g.dcase.layers[0]
    qv, qs = L.q(q_format)
    _say(f"[cfg5-{q_format}] dense")
    idx.idx_dense_masked_logits_topk(g.cfg, g.rows, ctx, qv, qs, L.weights, g.kcaches[0],
                                     g.sched.struct, dout, dout.stride(0), dlog, dlog.stride(0))
    torch.cuda.synchronize()
    dout_np = dout.cpu().numpy()
    np.testing.assert_array_equal(dout_np, res["indices"], err_msg="dense != sparse indices")
    dl = dlog.cpu().numpy()
    for i in range(R):
        gt, gl = gpu_row_tokens(res["sparse_indices"][i], int(res["kept"][i]), g.sbk, 0, ctx,
                                res["logits"][i])
        np.testing.assert_array_equal(dl[i, gt].view(np.uint32), gl.view(np.uint32),
                                      err_msg=f"dense logits differ bitwise row {i}")
    # the dense output against the oracle directly: its indices, and its logits read at
    # the schedule's candidate columns
    ncols = case.spec.nb * case.spec.cbs
    cols = np.arange(ncols)
    toks = res["sparse_indices"][:, cols // g.sbk].astype(np.int64) * g.sbk + cols % g.sbk
    dense_at_cols = np.take_along_axis(dl, np.clip(toks, 0, ctx - 1), axis=1)
    res_d = dict(res, indices=dout_np, logits=np.where(toks >= 0, dense_at_cols, -np.inf))
    ora = oracle.indexer_rows(case, 0, None, q_format, threads=THREADS)
    compare_rows(case, res_d, ora, case.spec.topk, g.sbk, f"cfg5-{q_format} dense")
    # the workspace form of the dense call gives the same indices
    ws = torch.empty(idx.idx_workspace_bytes(g.cfg, R, ctx), dtype=torch.uint8, device=DEV)
    dout.fill_(-7)
    idx.idx_dense_masked_logits_topk(g.cfg, g.rows, ctx, qv, qs, L.weights, g.kcaches[0],
                                     g.sched.struct, dout, dout.stride(0), None, 0, ws, ws.numel())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dout.cpu().numpy(), res["indices"])


@pytest.mark.parametrize("q_format", ["mxfp4", "fp8"])
@pytest.mark.parametrize("page_size", [16, 32])
def test_dense_comparator_on_small_pages(page_size, q_format):
    """The dense comparator on pages shorter than a 64-token group (each group spans
    several pages, so tiles are resolved one by one): the same indices as the sparse path
    (checked against the oracle on every row) and logits bitwise equal at the candidate
    tokens."""
    import sparse_attention_indexer_candidate_amd as idx

    spec = W.Spec(name=f"dp{page_size}", num_rows=24, page_size=page_size, cbs=page_size,
                  nb=40, topk=100, ke_rule="uniform", ke_lo=100, ke_hi=2000, ks_rule="random",
                  cand_rule="messy", fill="all", q_formats=("mxfp4", "fp8"))
    case = W.generate(spec, seed=13)
    g, res = run_and_compare(case, tag=f"dense-p{page_size}-{q_format}", q_format=q_format)
    R = case.num_rows
    ctx = int(case.row_ke.max())
    lstride = (ctx + 63) // 64 * 64
    dlog = torch.empty((R, lstride), dtype=torch.float32, device=DEV)
    dout = torch.full((R, spec.topk), -7, dtype=torch.int32, device=DEV)
    L = g.dcase.layers[0]
    qv, qs = L.q(q_format)
    idx.idx_dense_masked_logits_topk(g.cfg, g.rows, ctx, qv, qs, L.weights, g.kcaches[0],
                                     g.sched.struct, dout, dout.stride(0), dlog, dlog.stride(0))
    torch.cuda.synchronize()
    dout_np, dl = dout.cpu().numpy(), dlog.cpu().numpy()
    np.testing.assert_array_equal(dout_np, res["indices"], err_msg="dense != sparse indices")
    for i in range(R):
        gt, gl = gpu_row_tokens(res["sparse_indices"][i], int(res["kept"][i]), g.sbk,
                                int(case.row_ks[i]), int(case.row_ke[i]), res["logits"][i])
        np.testing.assert_array_equal(dl[i, gt].view(np.uint32), gl.view(np.uint32),
                                      err_msg=f"dense logits differ bitwise row {i}")


@pytest.mark.parametrize("name", ["split", "one_row", "row_groups"])
def test_range_edges_and_strides(name):
    """Rows with ks < 0, ks past ke, ke = 0 and ke < 0 (the empty and full readings of
    [ks, ke)), candidate arrays with a wider stride whose padding holds valid-looking ids
    (never read), and output rows wider than k (slots past k untouched): the schedule,
    logits and indices against the oracle on every row."""
    import dataclasses

    spec = DROPPED[name]
    case = W.generate(spec, seed=31)
    rng = np.random.default_rng(4)
    ks, ke = case.row_ks.copy(), case.row_ke.copy()
    r = rng.permutation(case.num_rows)
    ks[r[0:4]] = -5                                  # every token from 0
    ks[r[4:8]] = ke[r[4:8]] + 10                     # ks past ke: empty
    ks[r[8:10]] = np.maximum(ke[r[8:10]] - 1, 0)     # one token
    ke[r[10:12]] = 0
    ke[r[12:14]] = -3
    case = dataclasses.replace(case, row_ks=ks.astype(np.int32), row_ke=ke.astype(np.int32))
    d = to_device(case, DEV)
    R, nb, k = case.num_rows, spec.nb, spec.topk
    padded = torch.from_numpy(np.concatenate(
        [case.candidate_blocks, np.tile(np.arange(5, dtype=np.int32), (R, 1))], axis=1)).to(DEV)
    d.candidate_blocks = padded[:, :nb]              # stride nb + 5
    g = GpuRun(case, d)
    wide = torch.full((R, k + 7), -7, dtype=torch.int32, device=DEV)
    g.out = wide[:, :k]                              # out_stride k + 7
    _say(f"[edges-{name}] rows={R} cand_stride={d.candidate_blocks.stride(0)} "
         f"out_stride={g.out.stride(0)}")
    g.expand()
    g.score(0)
    res = g.fetch()
    si_o, end_o = oracle.expand(case, g.sbk)
    np.testing.assert_array_equal(res["sparse_indices"], si_o, err_msg="schedule")
    np.testing.assert_array_equal(res["end"], end_o, err_msg="end")
    ora = oracle.indexer_rows(case, 0, None, "mxfp4", threads=THREADS)
    compare_rows(case, res, ora, k, g.sbk, f"edges-{name}")
    assert np.all(wide[:, k:].cpu().numpy() == -7), "wrote past k"
    assert np.all(res["indices"][r[4:8]] == -1) and np.all(res["indices"][r[10:14]] == -1)


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


@pytest.mark.parametrize("name", sorted(DROPPED))
def test_pages_outside_the_pool_and_invalid_table_rows_are_dropped(name):
    """Sparse blocks on pages outside the pool, and every block of a row whose table row is
    out of range, leave the schedule unread: the schedule, logits and indices equal the
    oracle's on the original tables with those candidate blocks removed.  The dense
    comparator on the same inputs gives the sparse indices, with -inf at every token of a
    dropped page and on the rows without a table."""
    import sparse_attention_indexer_candidate_amd as idx

    case = W.generate(DROPPED[name], seed=21)
    bad, clean, bad_rows, bad_pages = corrupt_tables(case, seed=5)
    s = case.spec
    tag = f"drop-{name}"
    _say(f"[{tag}] rows={bad.num_rows} corrupted entries={int(bad_pages.sum())} "
         f"bad rows={bad_rows.tolist()}")
    g = GpuRun(bad, to_device(bad, DEV))
    g.expand()
    g.score(0)
    res = g.fetch()
    si_o, end_o = oracle.expand(clean, g.sbk)
    np.testing.assert_array_equal(res["sparse_indices"], si_o, err_msg=f"{tag}: schedule")
    np.testing.assert_array_equal(res["end"], end_o, err_msg=f"{tag}: end")
    assert np.all(res["indices"][bad_rows] == -1) and np.all(res["end"][bad_rows] == 0)
    ora = oracle.indexer_rows(clean, 0, None, "mxfp4", threads=THREADS)
    compare_rows(clean, res, ora, s.topk, g.sbk, tag)
    if name != "split":
        return
    R = bad.num_rows
    ctx = int(bad.row_ke.max())
    lstride = (ctx + 63) // 64 * 64
    dlog = torch.empty((R, lstride), dtype=torch.float32, device=DEV)
    dout = torch.full((R, s.topk), -7, dtype=torch.int32, device=DEV)
    L = g.dcase.layers[0]
    qv, qs = L.q("mxfp4")
    _say(f"[{tag}] dense")
    idx.idx_dense_masked_logits_topk(g.cfg, g.rows, ctx, qv, qs, L.weights, g.kcaches[0],
                                     g.sched.struct, dout, dout.stride(0), dlog, dlog.stride(0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dout.cpu().numpy(), res["indices"], err_msg="dense != sparse")
    dl = dlog.cpu().numpy()
    assert np.all(dl[bad_rows, :ctx] == -np.inf)
    for r in range(R):
        if r in bad_rows:
            continue
        ks, ke = int(bad.row_ks[r]), int(bad.row_ke[r])
        toks = np.arange(ks, ke)
        dropped = bad_pages[bad.row_table[r], toks // s.page_size]
        assert np.all(dl[r, toks[dropped]] == -np.inf), f"{tag}: row {r} dropped page scored"
        assert np.all(np.isfinite(dl[r, toks[~dropped]])), f"{tag}: row {r} mapped token"


@pytest.mark.parametrize("name", sorted(DROPPED))
def test_separate_value_and_scale_pools(name):
    """The two-pointer K cache: the values and the scales copied into two separate pools,
    each with its own page stride (values padded by 256 bytes a page; scales by 3 bytes
    from an odd base, as byte loads allow), give the interleaved pool's schedule, logits
    and indices bit for bit; on the split shape also the dense comparator, the source
    publication and (with 4-byte aligned scale pages, as it requires) the K gather."""
    import sparse_attention_indexer_candidate_amd as idx

    spec = DROPPED[name]
    case = W.generate(spec, seed=17)
    d = to_device(case, DEV)
    g = GpuRun(case, d)
    g.expand()
    g.score(0)
    ref = g.fetch()
    ps, pool, bt = spec.page_size, d.layers[0].pool, d.block_table
    P = pool.shape[0]
    vals = torch.zeros((P, ps * 64 + 256), dtype=torch.uint8, device=DEV)
    vals[:, :ps * 64] = pool[:, :ps * 64]
    sstride = ps * 4 + 3
    sbuf = torch.zeros(P * sstride + 64, dtype=torch.uint8, device=DEV)
    torch.as_strided(sbuf, (P, ps * 4), (sstride, 1), 1).copy_(pool[:, ps * 64:])
    k_split = idx.idx_kcache(vals.data_ptr(), vals.stride(0), sbuf.data_ptr() + 1, sstride, P,
                             bt.data_ptr(), bt.stride(0), bt.shape[0], bt.shape[1])
    k_ref = g.kcaches[0]
    g.kcaches[0] = k_split
    _say(f"[pools-{name}] rows={case.num_rows} values stride {vals.stride(0)} scales stride "
         f"{sstride}")
    g.out.fill_(-7)
    g.expand()
    g.score(0)
    res = g.fetch()
    for key in ("sparse_indices", "end", "indices"):
        np.testing.assert_array_equal(res[key], ref[key], err_msg=f"pools-{name}: {key}")
    np.testing.assert_array_equal(res["logits"].view(np.uint32), ref["logits"].view(np.uint32))
    if name != "split":
        return
    R, k = case.num_rows, spec.topk
    L = d.layers[0]
    qv, qs = L.q("mxfp4")
    ctx = int(case.row_ke.max())
    lstride = (ctx + 63) // 64 * 64
    dense = []
    for kc in (k_ref, k_split):
        dlog = torch.empty((R, lstride), dtype=torch.float32, device=DEV)
        dout = torch.full((R, k), -7, dtype=torch.int32, device=DEV)
        idx.idx_dense_masked_logits_topk(g.cfg, g.rows, ctx, qv, qs, L.weights, kc,
                                         g.sched.struct, dout, dout.stride(0), dlog,
                                         dlog.stride(0))
        dense.append((dout, dlog))
    pub = []
    ws = torch.empty(max(4, idx.idx_publish_workspace_bytes(g.cfg, R, ctx)), dtype=torch.uint8,
                     device=DEV)
    for kc in (k_ref, k_split):
        cand = torch.full((R, spec.nb), -7, dtype=torch.int32, device=DEV)
        plog = torch.empty((R, lstride), dtype=torch.float32, device=DEV)
        idx.idx_publish_candidates(g.cfg, g.rows, ctx, qv, qs, L.weights, kc, cand,
                                   cand.stride(0), plog, plog.stride(0), ws, ws.numel())
        torch.cuda.synchronize()
        pub.append((cand.cpu().numpy(), plog.cpu().numpy()))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dense[1][0].cpu().numpy(), dense[0][0].cpu().numpy())
    np.testing.assert_array_equal(dense[1][1].cpu().numpy().view(np.uint32),
                                  dense[0][1].cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(pub[1][0], pub[0][0])
    np.testing.assert_array_equal(pub[1][1].view(np.uint32), pub[0][1].view(np.uint32))
    # the gather reads a position's scale bytes as one word: 4-byte aligned scale pages
    sstride4 = ps * 4 + 4
    sbuf4 = torch.zeros((P, sstride4), dtype=torch.uint8, device=DEV)
    sbuf4[:, :ps * 4] = pool[:, ps * 64:]
    k_split4 = idx.idx_kcache(vals.data_ptr(), vals.stride(0), sbuf4.data_ptr(), sstride4, P,
                              bt.data_ptr(), bt.stride(0), bt.shape[0], bt.shape[1])
    lens = case.row_ke.astype(np.int64)
    cu = torch.from_numpy(np.r_[0, np.cumsum(lens)].astype(np.int32)).to(DEV)
    n = int(lens.sum())
    got = []
    for kc in (k_ref, k_split4):
        gv = torch.full((n, 64), 0xAB, dtype=torch.uint8, device=DEV)
        gs = torch.full((n, 4), 0xAB, dtype=torch.uint8, device=DEV)
        idx.idx_gather_k_workspace(g.cfg, kc, cu, gv, gs, int(lens.max()))
        torch.cuda.synchronize()
        got.append((gv.cpu().numpy(), gs.cpu().numpy()))
    np.testing.assert_array_equal(got[1][0], got[0][0])
    np.testing.assert_array_equal(got[1][1], got[0][1])


# Launch forms that no other case reaches, each named by what it takes
WIDE_FORMS = {
    # the dense comparator's selection with 16 keys a thread (over 4096 candidate columns)
    "dense_8192_columns": W.Spec(name="wf1", num_rows=24, page_size=64, cbs=64, nb=128,
                                 topk=3000, ke_rule="uniform", ke_lo=8000, ke_hi=14000,
                                 ks_rule="random", cand_rule="distinct", fill="all"),
    # row groups for 8192-column rows: two layers in one launch, and bf16 scoring
    "row_groups_8192_layers": W.Spec(name="wf2", num_rows=2048, page_size=64, cbs=64, nb=100,
                                     topk=1000, layers=2, mode="prefill", ke_rule="uniform",
                                     ke_lo=1, ke_hi=6400, ks_rule="random", context=6400,
                                     cand_rule="messy", fill="all"),
    "row_groups_8192_bf16": W.Spec(name="wf3", num_rows=2048, page_size=64, cbs=64, nb=100,
                                   topk=1000, mode="prefill", ke_rule="uniform", ke_lo=1,
                                   ke_hi=6400, context=6400, cand_rule="causal_all", fill="all"),
    # two 8-wave rows a CU with 16 keys a thread on 32-token sparse blocks
    "one_row_two_a_cu_sbk32_16_keys": W.Spec(name="wf4", num_rows=520, page_size=32, cbs=32,
                                             nb=200, topk=1500, ke_rule="uniform", ke_lo=2000,
                                             ke_hi=9000, ks_rule="random", cand_rule="messy",
                                             fill="all"),
}


@pytest.mark.parametrize("name", sorted(WIDE_FORMS))
def test_wide_launch_forms_all_rows(name):
    import sparse_attention_indexer_candidate_amd as idx

    spec = WIDE_FORMS[name]
    case = W.generate(spec, seed=23)
    if name == "row_groups_8192_layers":
        _check_layers_call(case, name, "mxfp4")
        return
    sf = "bf16" if name.endswith("bf16") else "fp32"
    g, res = run_and_compare(case, tag=name, score_format=sf)
    if name == "dense_8192_columns":
        ctx = int(case.row_ke.max() + 63) // 64 * 64
        assert idx.idx_num_sparse_blocks(g.cfg) * g.sbk > 4096
        np.testing.assert_array_equal(_dense_indices(g, case, ctx), res["indices"],
                                      err_msg="dense != sparse indices")


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


# (query format, score format, spec): every instantiation of the one-row, multi-layer and
# row-group kernels that the other cases leave out, by row count (one or two rows a CU,
# 8- or 4-wave fp8 rows), width (4 to 32 keys a thread) and sparse block (64, or 32: the
# per-tile path)
KERNEL_SWEEP = {
    "mx_layers_two_a_cu_8keys_sbk32": ("mxfp4", "fp32", _sweep_spec("k1", 260, 32, 100, 2)),
    "mx_rows_two_a_cu_8keys_sbk64": ("mxfp4", "fp32", _sweep_spec("k2", 520, 64, 50)),
    "mx_rows_two_a_cu_8keys_sbk32": ("mxfp4", "fp32", _sweep_spec("k3", 520, 32, 100)),
    "f8_layers_4wave_4keys_sbk32": ("fp8", "fp32", _sweep_spec("k4", 260, 32, 20, 2)),
    "f8_layers_4wave_8keys_sbk32": ("fp8", "fp32", _sweep_spec("k5", 260, 32, 50, 2)),
    "f8_layers_4wave_16keys_sbk32": ("fp8", "fp32", _sweep_spec("k6", 260, 32, 100, 2)),
    "f8_layers_4wave_32keys_sbk32": ("fp8", "fp32", _sweep_spec("k7", 260, 32, 200, 2)),
    "f8_layers_8wave_4keys_sbk32": ("fp8", "fp32", _sweep_spec("k8", 150, 32, 40, 2)),
    "f8_layers_8wave_8keys_sbk32": ("fp8", "fp32", _sweep_spec("k9", 150, 32, 100, 2)),
    "f8_layers_8wave_8keys_sbk64": ("fp8", "fp32", _sweep_spec("k10", 150, 64, 50, 2)),
    "f8_layers_8wave_16keys_sbk64": ("fp8", "fp32", _sweep_spec("k11", 150, 64, 100, 2)),
    "f8_rows_4wave_4keys_sbk32": ("fp8", "fp32", _sweep_spec("k12", 520, 32, 20)),
    "f8_rows_4wave_8keys_sbk32": ("fp8", "fp32", _sweep_spec("k13", 520, 32, 50)),
    "f8_rows_4wave_8keys_sbk64": ("fp8", "fp32", _sweep_spec("k14", 520, 64, 25)),
    "f8_rows_4wave_16keys_sbk32": ("fp8", "fp32", _sweep_spec("k15", 520, 32, 100)),
    "f8_rows_4wave_32keys_sbk32": ("fp8", "fp32", _sweep_spec("k16", 520, 32, 200)),
    "f8_rows_8wave_8keys_sbk32": ("fp8", "fp32", _sweep_spec("k17", 300, 32, 100)),
    "bf16_row_group_layers_4096": ("mxfp4", "bf16", _sweep_spec("k18", 2048, 64, 60, 2, True)),
    "bf16_row_group_layers_8192": ("mxfp4", "bf16", _sweep_spec("k19", 2048, 64, 100, 2, True)),
}


@pytest.mark.parametrize("name", sorted(KERNEL_SWEEP))
def test_kernel_instantiation_sweep(name):
    """One case per launch form: single-layer calls against the oracle on every row;
    multi-layer calls also against one call per layer, bit for bit."""
    q_format, score_format, spec = KERNEL_SWEEP[name]
    case = W.generate(spec, seed=29)
    _say(f"[sweep-{name}] rows={spec.num_rows} cbs={spec.cbs} nb={spec.nb} layers={spec.layers}")
    if spec.layers > 1:
        _check_layers_call(case, name, q_format, score_format)
    else:
        run_and_compare(case, tag=name, q_format=q_format, score_format=score_format)


LAYERED = {
    # >= 256 rows of one table row each: every layer in one launch
    "one_launch": W.Spec(name="ml1", num_rows=300, page_size=64, cbs=64, nb=24, topk=300,
                         layers=3, ke_rule="uniform", ke_lo=500, ke_hi=3000, ks_rule="random",
                         cand_rule="messy", fill="all", q_formats=("mxfp4", "fp8")),
    # the layer limit (8) in one launch
    "eight_layers": W.Spec(name="ml3", num_rows=260, page_size=64, cbs=64, nb=8, topk=100,
                           layers=8, ke_rule="uniform", ke_lo=10, ke_hi=1500, cand_rule="messy",
                           fill="all", q_formats=("mxfp4", "fp8")),
    # >= 8 rows per CU on one table (a prefill chunk's shape): row groups, layer by layer
    "row_groups": W.Spec(name="ml4", num_rows=2050, page_size=128, cbs=64, nb=8, topk=100,
                         layers=2, mode="prefill", ke_rule="uniform", ke_lo=1, ke_hi=1500,
                         ks_rule="random", context=1600, cand_rule="messy", fill="all",
                         q_formats=("mxfp4", "fp8")),
    # 4096-column rows in one launch (8 keys a thread at 512 threads)
    "one_launch_4096": W.Spec(name="ml5", num_rows=260, page_size=64, cbs=64, nb=64, topk=2048,
                              layers=2, ke_rule="uniform", ke_lo=3000, ke_hi=9000,
                              cand_rule="distinct", fill="candidates"),
    # fewer rows than CUs at the column and top-k limits: the batched split selection
    # with 16 keys a thread
    "split_wide": W.Spec(name="ml6", num_rows=24, page_size=64, cbs=64, nb=128, topk=7000,
                         layers=2, ke_rule="uniform", ke_lo=6000, ke_hi=12000,
                         cand_rule="distinct", fill="candidates"),
    # fewer rows than CUs but more row-layers: one workgroup a row-layer in one launch
    "row_layers": W.Spec(name="ml7", num_rows=40, page_size=64, cbs=64, nb=16, topk=300,
                         layers=8, ke_rule="uniform", ke_lo=10, ke_hi=1200, cand_rule="messy",
                         fill="all", q_formats=("mxfp4", "fp8")),
    # two row-layers a CU at the column limit: fp8 queries take 4-wave rows with 32 keys a
    # thread (sbk 64)
    "wide_two_rows_a_cu": W.Spec(name="ml8", num_rows=260, page_size=64, cbs=64, nb=128,
                                 topk=2048, layers=2, ke_rule="uniform", ke_lo=6000,
                                 ke_hi=12000, cand_rule="distinct", fill="candidates"),
    # ... and with 16-token sparse blocks, too short for 32 keys a thread: 8-wave rows
    "wide_sbk16": W.Spec(name="ml9", num_rows=260, page_size=32, cbs=16, nb=320, topk=1000,
                         layers=2, ke_rule="uniform", ke_lo=3000, ke_hi=9000,
                         cand_rule="messy", fill="candidates"),
    # fewer rows than CUs: the split kernels, layer after layer
    "split": W.Spec(name="ml2", num_rows=40, page_size=32, cbs=32, nb=30, topk=500, layers=2,
                    ke_rule="uniform", ke_lo=100, ke_hi=1500, cand_rule="messy", fill="all",
                    q_formats=("mxfp4", "fp8")),
}


@pytest.mark.parametrize("q_format", ["mxfp4", "fp8"])
@pytest.mark.parametrize("name", sorted(LAYERED))
def test_layers_call_matches_per_layer_calls_and_oracle(name, q_format):
    import dataclasses

    spec = LAYERED[name]
    if q_format not in spec.q_formats:
        spec = dataclasses.replace(spec, q_formats=("mxfp4", "fp8"))
    _check_layers_call(W.generate(spec, seed=5), name, q_format)


@pytest.mark.parametrize("i", range(10))
def test_random_layers_calls(i):
    """Seeded random multi-layer calls: 2-8 layers, row counts that take each multi-layer
    form (batched split launches, one launch of row-layers, two fp8 row-layers a CU, row
    groups), random block and page sizes and k; the same checks as the fixed cases."""
    import dataclasses

    rng = np.random.default_rng(7000 + i)
    spec, _ = _random_spec(200 + i)
    layers = int(rng.integers(2, 9))
    form = i % 4
    rows = [int(rng.integers(8, 256 // layers)), int(rng.integers(256 // layers + 1, 255)),
            int(rng.integers(256, 400)), spec.num_rows][form]
    if form == 3 and spec.mode != "prefill":
        spec = dataclasses.replace(spec, mode="prefill", ke_lo=1, context=spec.ke_hi)
        rows = 2048 + int(rng.integers(0, 40))
    spec = dataclasses.replace(spec, name=f"rl{i}", num_rows=rows, layers=layers,
                               q_formats=("mxfp4", "fp8"))
    q_format = ("mxfp4", "fp8")[(i + i // 4) % 2]   # each form with both formats
    _say(f"[rl{i}] rows={rows} layers={layers} cbs={spec.cbs} page={spec.page_size} "
         f"nb={spec.nb} k={spec.topk} {spec.mode} {q_format}")
    _check_layers_call(W.generate(spec, seed=70 + i), f"rl{i}", q_format)


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


def test_layers_call_on_long_decode_matches_per_layer_calls():
    """The timed form of the long-context decode step: one multi-layer call for the four
    layers (one launch), every row of every layer against the oracle, and bit for bit
    against one call per layer."""
    case = W.generate(W.config(4), 0)
    g = GpuRun(case, to_device(case, DEV))
    g.expand()
    _say("[layers-cfg4] one call, 4 layers")
    outs, logs = g.score_layers(range(4), [True, False, False, True])
    torch.cuda.synchronize()
    for layer in range(4):
        _say(f"[layers-cfg4] layer {layer}")
        g.out.fill_(-7)
        g.score(layer, with_logits=True)
        res = g.fetch()
        np.testing.assert_array_equal(outs[layer].cpu().numpy(), res["indices"],
                                      err_msg=f"cfg4 layer {layer}: indices")
        if logs[layer] is not None:
            np.testing.assert_array_equal(logs[layer].cpu().numpy().view(np.uint32),
                                          res["logits"].view(np.uint32))
        pool = case.layers[layer].host_pool(case.spec.page_bytes)
        ora = oracle.indexer_rows(case, layer, None, "mxfp4", pool=pool, threads=THREADS)
        res["indices"] = outs[layer].cpu().numpy()
        compare_rows(case, res, ora, case.spec.topk, g.sbk, f"layers-cfg4 layer {layer}")
    # one layer through the multi-layer entry point takes the one-layer launch
    one, _ = g.score_layers([3], [False])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(one[0].cpu().numpy(), outs[3].cpu().numpy(),
                                  err_msg="cfg4 one layer")


def test_repeat_calls_are_deterministic_and_reuse_schedule():
    case = W.generate(W.config(2), 1)
    dcase = to_device(case, DEV)
    g = GpuRun(case, dcase)
    g.expand()
    g.score(0)
    a = g.fetch()
    for _ in range(3):
        g.out.fill_(-7)
        g.score(0)
        b = g.fetch()
        np.testing.assert_array_equal(a["indices"], b["indices"])
        np.testing.assert_array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))


def test_invariances_page_permutation_scale_and_weights():
    spec = W.Spec(name="inv", num_rows=8, page_size=64, cbs=64, nb=16, topk=200,
                  ke_rule="uniform", ke_lo=1500, ke_hi=4000, cand_rule="messy", fill="all")
    case = W.generate(spec, seed=9)
    g0, r0 = run_and_compare(case, tag="inv-base")
    # permuting the physical pages (data and block table together) changes nothing
    L = case.layers[0]
    perm = np.random.default_rng(1).permutation(L.num_pages)
    case_p = W.Case(spec, 9, case.row_ks, case.row_ke, case.row_table,
                    np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32),
                    case.candidate_blocks,
                    [W.LayerData(L.weights, L.num_pages, perm[L.filled_pages], L.filled_data,
                                 L.q_values, L.q_scales)])
    g1, r1 = run_and_compare(case_p, tag="inv-perm")
    np.testing.assert_array_equal(r0["indices"], r1["indices"])
    np.testing.assert_array_equal(r0["logits"].view(np.uint32), r1["logits"].view(np.uint32))
    # every K scale byte + 1 doubles every logit exactly and keeps the indices
    data2 = L.filled_data.copy()
    data2[:, spec.values_bytes:] += 1
    case_s = W.Case(spec, 9, case.row_ks, case.row_ke, case.row_table, case.block_table,
                    case.candidate_blocks,
                    [W.LayerData(L.weights, L.num_pages, L.filled_pages, data2, L.q_values, L.q_scales)])
    g2, r2 = run_and_compare(case_s, tag="inv-scale")
    np.testing.assert_array_equal(r0["indices"], r2["indices"])
    fin = np.isfinite(r0["logits"])
    np.testing.assert_array_equal(r2["logits"][fin], 2 * r0["logits"][fin])
    # shuffled candidate order gives the same schedule and result
    cand = case.candidate_blocks.copy()
    for r in range(cand.shape[0]):
        cand[r] = np.random.default_rng(r).permutation(cand[r])
    case_c = W.Case(spec, 9, case.row_ks, case.row_ke, case.row_table, case.block_table, cand,
                    case.layers)
    g3, r3 = run_and_compare(case_c, tag="inv-shuffle")
    np.testing.assert_array_equal(r0["indices"], r3["indices"])
    np.testing.assert_array_equal(r0["logits"].view(np.uint32), r3["logits"].view(np.uint32))


@pytest.mark.parametrize("which", ["decode_batch", "rows_per_cu"])
def test_step_graph_replays_match_eager(which):
    """A step (expansion, sparse scoring and the dense comparator) captured as one HIP
    graph on its own stream and replayed several times, with eager steps of other
    inputs on the same stream between the replays: every replay gives the eager
    result, bit for bit (the library records no memset and allocates nothing)."""
    import sparse_attention_indexer_candidate_amd as idx

    spec = W.config(2) if which == "decode_batch" else WEIGHT_PATHS["fused"]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        sh = stream.cuda_stream
        runs = []
        for seed in (0, 1):
            case = W.generate(spec, seed)
            d = to_device(case, DEV)
            s = case.spec
            cfg = idx.make_config(s.num_heads, s.head_dim, idx.IDX_Q_MXFP4, s.page_size, s.cbs, 0,
                                  s.nb, s.topk)
            R = case.num_rows
            ctx = int(case.row_ke.max() + 63) // 64 * 64
            rows = idx.make_rows(d.row_ke, d.row_ks, d.row_table)
            kc = idx.make_kcache(d.layers[0].pool, s.page_size, s.head_dim, d.block_table)
            sched = idx.Schedule(cfg, R, DEV)
            out = torch.full((R, s.topk), -7, dtype=torch.int32, device=DEV)
            dout = torch.full((R, s.topk), -7, dtype=torch.int32, device=DEV)
            ws = torch.empty(idx.idx_workspace_bytes(cfg, R, ctx), dtype=torch.uint8, device=DEV)
            qv, qs = d.layers[0].q("mxfp4")
            calls = [idx.bind_expand_candidates(cfg, rows, kc, d.candidate_blocks,
                                                d.candidate_blocks.stride(0), sched.struct,
                                                stream=sh),
                     idx.bind_sparse_mqa_logits_topk(cfg, rows, qv, qs, d.layers[0].weights, kc,
                                                     sched.struct, out, out.stride(0), None, ws,
                                                     ws.numel(), stream=sh),
                     idx.bind_dense_masked_logits_topk(cfg, rows, ctx, qv, qs,
                                                       d.layers[0].weights, kc, sched.struct, dout,
                                                       dout.stride(0), None, 0, ws, ws.numel(),
                                                       stream=sh)]
            runs.append(dict(keep=(d, rows, kc, sched, ws), calls=calls, out=out, dout=dout))
        for r in runs:                                   # eager results
            for c in r["calls"]:
                c()
        torch.cuda.synchronize()
        for r in runs:
            r["ref"], r["dref"] = r["out"].clone(), r["dout"].clone()
        np.testing.assert_array_equal(runs[0]["ref"].cpu().numpy(), runs[0]["dref"].cpu().numpy())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in runs[0]["calls"]:
                c()
        other = runs[1]
        for rep in range(3):
            runs[0]["out"].fill_(-7)
            runs[0]["dout"].fill_(-7)
            other["out"].fill_(-7)
            for c in other["calls"]:                     # eager work between replays
                c()
            g.replay()
            torch.cuda.synchronize()
            _say(f"[graph {which}] replay {rep}")
            assert torch.equal(runs[0]["out"], runs[0]["ref"]), f"replay {rep}: sparse indices"
            assert torch.equal(runs[0]["dout"], runs[0]["dref"]), f"replay {rep}: dense indices"
            assert torch.equal(other["out"], other["ref"]), f"replay {rep}: eager step"


def test_gather_k_workspace_matches_oracle():
    """Several requests (one empty), each through another row's table, an out-of-range
    page id, a row cap below the total: the packed workspace byte for byte."""
    import sparse_attention_indexer_candidate_amd as idx

    spec = W.Spec(name="gather", num_rows=7, page_size=64, cbs=64, nb=4, topk=64,
                  ke_rule="uniform", ke_lo=0, ke_hi=5000, cand_rule="distinct", fill="all")
    case = W.generate(spec, seed=3)
    lens = case.row_ke.astype(np.int64)
    lens[4] = 0
    cu = np.r_[0, np.cumsum(lens)].astype(np.int32)
    req = np.ascontiguousarray(case.row_table[::-1]).astype(np.int32)
    bt = case.block_table.copy()
    bt[req[int(np.argmax(lens))], 1] = 1 << 24             # no such page: zeros
    max_tokens, max_seq = int(cu[-1]) - 50, int(lens.max())
    pool = case.layers[0].host_pool(spec.page_bytes)
    want_v, want_s = oracle.gather_k_workspace(pool, spec.page_size, spec.head_dim, bt, cu,
                                               req_table=req, max_seq_len=max_seq,
                                               max_tokens=max_tokens, fill=0xAB)
    d = to_device(case, DEV)
    dbt = torch.from_numpy(bt).to(DEV)
    cfg = idx.make_config(64, 128, idx.IDX_Q_MXFP4, spec.page_size, spec.cbs, 0, spec.nb, spec.topk)
    kc = idx.make_kcache(d.layers[0].pool, spec.page_size, spec.head_dim, dbt)
    vals = torch.full((max_tokens, 64), 0xAB, dtype=torch.uint8, device=DEV)
    scs = torch.full((max_tokens, 4), 0xAB, dtype=torch.uint8, device=DEV)
    _say(f"[gather] {len(lens)} requests, {max_tokens} rows")
    idx.idx_gather_k_workspace(cfg, kc, torch.from_numpy(cu).to(DEV), vals, scs, max_seq,
                               req_table=torch.from_numpy(req).to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(vals.cpu().numpy(), want_v)
    np.testing.assert_array_equal(scs.cpu().numpy(), want_s)
    # no request table: request r reads table row r
    want_v, want_s = oracle.gather_k_workspace(pool, spec.page_size, spec.head_dim, bt, cu,
                                               max_seq_len=max_seq, max_tokens=max_tokens,
                                               fill=0x5C)
    vals.fill_(0x5C)
    scs.fill_(0x5C)
    idx.idx_gather_k_workspace(cfg, kc, torch.from_numpy(cu).to(DEV), vals, scs, max_seq)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(vals.cpu().numpy(), want_v)
    np.testing.assert_array_equal(scs.cpu().numpy(), want_s)


@pytest.mark.parametrize("i", range(10))
def test_random_gathers(i):
    """Seeded random gathers, byte for byte against the oracle: page sizes 16-256, 1-40
    requests (some empty), request tables with rows out of range, page ids outside the
    pool, and caps on the sequence length and on the workspace rows."""
    import sparse_attention_indexer_candidate_amd as idx

    rng = np.random.default_rng(8000 + i)
    page_size = (16, 32, 64, 128, 256)[i % 5]
    cbs = min(64, page_size)
    nreq = int(rng.integers(1, 41))
    spec = W.Spec(name=f"rg{i}", num_rows=nreq, page_size=page_size, cbs=cbs, nb=4, topk=16,
                  ke_rule="uniform", ke_lo=0, ke_hi=int(rng.integers(1, 6000)),
                  cand_rule="distinct", fill="all")
    case = W.generate(spec, seed=80 + i)
    lens = case.row_ke.astype(np.int64)
    lens[rng.random(nreq) < 0.15] = 0
    cu = np.r_[0, np.cumsum(lens)].astype(np.int32)
    T = case.block_table.shape[0]
    req = rng.permutation(T)[:nreq].astype(np.int32) if T >= nreq else \
        rng.integers(0, T, nreq).astype(np.int32)
    bad = rng.random(nreq) < 0.1
    req[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, T).astype(np.int32)
    bt = case.block_table.copy()
    live = np.argwhere(bt >= 0)
    if len(live):
        pick = live[rng.choice(len(live), size=max(1, len(live) // 10), replace=False)]
        bt[pick[:, 0], pick[:, 1]] = np.where(rng.random(len(pick)) < 0.5, -1,
                                              case.layers[0].num_pages + 7)
    total = int(cu[-1])
    max_seq = max(1, int(lens.max()) - int(rng.integers(0, 2) * rng.integers(0, 300)))
    max_tokens = max(1, total - int(rng.integers(0, 2) * rng.integers(0, 500)))
    pool = case.layers[0].host_pool(spec.page_bytes)
    want_v, want_s = oracle.gather_k_workspace(pool, page_size, spec.head_dim, bt, cu,
                                               req_table=req, max_seq_len=max_seq,
                                               max_tokens=max_tokens, fill=0xAB)
    d = to_device(case, DEV)
    # every device array the launch reads stays referenced until it has finished (the
    # K-cache struct holds only the table's address)
    dbt, dcu, dreq = (torch.from_numpy(a).to(DEV) for a in (bt, cu, req))
    cfg = idx.make_config(64, 128, idx.IDX_Q_MXFP4, page_size, cbs, 0, spec.nb, spec.topk)
    kc = idx.make_kcache(d.layers[0].pool, page_size, spec.head_dim, dbt)
    vals = torch.full((max_tokens, 64), 0xAB, dtype=torch.uint8, device=DEV)
    scs = torch.full((max_tokens, 4), 0xAB, dtype=torch.uint8, device=DEV)
    _say(f"[rg{i}] page={page_size} requests={nreq} positions={total} max_seq={max_seq} "
         f"rows={max_tokens} bad tables={int(bad.sum())}")
    idx.idx_gather_k_workspace(cfg, kc, dcu, vals, scs, max_seq, req_table=dreq)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(vals.cpu().numpy(), want_v)
    np.testing.assert_array_equal(scs.cpu().numpy(), want_s)


def test_gather_then_score_equals_paged_cache():
    """A prefill chunk scored from its gathered workspace (one page of 2048 positions)
    gives the paged cache's indices and logits bit for bit."""
    import sparse_attention_indexer_candidate_amd as idx

    n = 2048
    spec = W.Spec(name="gws", num_rows=300, page_size=64, cbs=64, nb=16, topk=128,
                  mode="prefill", ke_rule="uniform", ke_lo=1, ke_hi=n, ks_rule="random",
                  context=n, cand_rule="messy", fill="all")
    case = W.generate(spec, seed=4)
    g = GpuRun(case, to_device(case, DEV))
    g.expand()
    g.score(0, with_logits=True)
    ref = g.fetch()
    d = g.dcase
    vals = torch.empty((n, 64), dtype=torch.uint8, device=DEV)
    scs = torch.empty((n, 4), dtype=torch.uint8, device=DEV)
    _say("[gather-score] gather")
    idx.idx_gather_k_workspace(g.cfg, g.kcaches[0], torch.tensor([0, n], dtype=torch.int32,
                                                                 device=DEV), vals, scs, n,
                               req_table=d.row_table[:1])
    wcfg = idx.make_config(64, 128, idx.IDX_Q_MXFP4, n, spec.cbs, 0, spec.nb, spec.topk)
    wbt = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    wk = idx.make_workspace_kcache(vals, scs, wbt)
    R = case.num_rows
    rows = idx.make_rows(d.row_ke, d.row_ks, torch.zeros(R, dtype=torch.int32, device=DEV))
    sched = idx.Schedule(wcfg, R, DEV)
    idx.idx_expand_candidates(wcfg, rows, wk, d.candidate_blocks, d.candidate_blocks.stride(0),
                              sched.struct)
    out = torch.full((R, spec.topk), -7, dtype=torch.int32, device=DEV)
    lg = torch.empty((R, spec.nb * spec.cbs), dtype=torch.float32, device=DEV)
    qv, qs = d.layers[0].q("mxfp4")
    _say("[gather-score] score the workspace")
    idx.idx_sparse_mqa_logits_topk(wcfg, rows, qv, qs, d.layers[0].weights, wk, sched.struct, out,
                                   out.stride(0), lg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), ref["indices"])
    np.testing.assert_array_equal(lg.cpu().numpy().view(np.uint32), ref["logits"].view(np.uint32))


@pytest.mark.parametrize("name", ["split", "one_launch"])
def test_layers_call_graph_replays_match_eager(name):
    """The expansion and one multi-layer call (every layer's logits in the workspace, so
    fewer rows than CUs take the batched split launches) captured as one HIP graph and
    replayed with eager steps of other inputs between the replays: every replay gives
    the eager indices of every layer."""
    import sparse_attention_indexer_candidate_amd as idx

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        sh = stream.cuda_stream
        runs = []
        for seed in (0, 1):
            case = W.generate(LAYERED[name], seed)
            d = to_device(case, DEV)
            s = case.spec
            R, nl = case.num_rows, s.layers
            cfg = idx.make_config(s.num_heads, s.head_dim, idx.IDX_Q_MXFP4, s.page_size, s.cbs, 0,
                                  s.nb, s.topk)
            rows = idx.make_rows(d.row_ke, d.row_ks, d.row_table)
            kcs = [idx.make_kcache(L.pool, s.page_size, s.head_dim, d.block_table) for L in d.layers]
            sched = idx.Schedule(cfg, R, DEV)
            outs = [torch.full((R, s.topk), -7, dtype=torch.int32, device=DEV) for _ in range(nl)]
            ws = torch.empty(idx.idx_workspace_bytes(cfg, R * nl, 0), dtype=torch.uint8, device=DEV)
            entries = [(*L.q("mxfp4"), L.weights, kcs[i], outs[i], None)
                       for i, L in enumerate(d.layers)]
            calls = [idx.bind_expand_candidates(cfg, rows, kcs[0], d.candidate_blocks,
                                                d.candidate_blocks.stride(0), sched.struct,
                                                stream=sh),
                     idx.bind_sparse_mqa_logits_topk_layers(cfg, rows, sched.struct, entries, s.topk,
                                                            ws, ws.numel(), stream=sh)]
            runs.append(dict(keep=(d, rows, kcs, sched, ws), calls=calls, outs=outs))
        for r in runs:                                   # eager results
            for c in r["calls"]:
                c()
        torch.cuda.synchronize()
        for r in runs:
            r["refs"] = [o.clone() for o in r["outs"]]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in runs[0]["calls"]:
                c()
        other = runs[1]
        for rep in range(3):
            for o in runs[0]["outs"] + other["outs"]:
                o.fill_(-7)
            for c in other["calls"]:                     # eager work between replays
                c()
            g.replay()
            torch.cuda.synchronize()
            _say(f"[graph layers {name}] replay {rep}")
            for layer, (o, ref) in enumerate(zip(runs[0]["outs"], runs[0]["refs"])):
                assert torch.equal(o, ref), f"replay {rep} layer {layer}"
            for layer, (o, ref) in enumerate(zip(other["outs"], other["refs"])):
                assert torch.equal(o, ref), f"eager between replays, layer {layer}"


# ---------------------------------------------------------------- bf16 scoring ----
# bf16 head weights and bf16-rounded logits (the SM100 layer's semantics): every kernel
# path against the oracle's bf16 scoring, every row.

BF16_PATHS = {
    "split": SMALL["ragged_sbk64_ks"],
    "split_sbk16": SMALL["sbk16"],
    "one_row": WEIGHT_PATHS["fused"],
    "two_rows_a_cu": SMALL["two_rows_a_cu"],
    "row_groups": SMALL["rowgroup_shared_table_messy"],
}


@pytest.mark.parametrize("path", sorted(BF16_PATHS))
def test_bf16_scoring_kernel_paths_all_rows(path):
    run_and_compare(W.generate(BF16_PATHS[path], seed=31), tag=f"bf16-{path}",
                    score_format="bf16")


def test_bf16_scoring_fp8_query():
    spec = W.Spec(name="bf8", num_rows=40, page_size=64, cbs=64, nb=12, topk=150,
                  ke_rule="uniform", ke_lo=10, ke_hi=2500, ks_rule="random", cand_rule="messy",
                  fill="all", q_formats=("mxfp4", "fp8"))
    run_and_compare(W.generate(spec, seed=6), q_format="fp8", tag="bf16-fp8", score_format="bf16")


def test_bf16_scoring_decode_batch_all_rows():
    run_and_compare(W.generate(W.config(2), 0), tag="bf16-cfg2", score_format="bf16")


def test_bf16_scoring_long_decode_layers_call_all_rows():
    """The long-context decode batch in bf16 scoring: one multi-layer call (one launch)
    for the four layers, each layer's indices equal to its own call's, every row of every
    layer against the oracle's bf16 scoring."""
    case = W.generate(W.config(4), 0)
    g = GpuRun(case, to_device(case, DEV), score_format="bf16")
    g.expand()
    _say("[bf16-cfg4] one call, 4 layers")
    outs, _ = g.score_layers(range(4), [False] * 4)
    torch.cuda.synchronize()
    for layer in range(4):
        _say(f"[bf16-cfg4] layer {layer}")
        g.out.fill_(-7)
        g.score(layer, with_logits=True)
        res = g.fetch()
        np.testing.assert_array_equal(outs[layer].cpu().numpy(), res["indices"],
                                      err_msg=f"bf16 cfg4 layer {layer}: one call != per layer")
        pool = case.layers[layer].host_pool(case.spec.page_bytes)
        ora = oracle.indexer_rows(case, layer, None, "mxfp4", pool=pool, threads=THREADS,
                                  score_format="bf16")
        compare_rows(case, res, ora, case.spec.topk, g.sbk, f"bf16-cfg4 layer {layer}",
                     score_format="bf16")


def test_bf16_scoring_prefill_chunk_all_rows():
    run_and_compare(W.generate(W.config(3), 0), tag="bf16-cfg3", score_format="bf16")


def test_bf16_scoring_dense_equals_sparse():
    """The dense comparator in bf16 scoring returns the sparse path's indices (the same
    per-column arithmetic and the same rounding)."""
    import sparse_attention_indexer_candidate_amd as idx

    case = W.generate(W.config(5), 0)
    g, res = run_and_compare(case, tag="bf16-cfg5", score_format="bf16")
    R, ctx = case.num_rows, 65536
    dout = torch.full((R, case.spec.topk), -7, dtype=torch.int32, device=DEV)
    dlog = torch.empty((R, ctx), dtype=torch.float32, device=DEV)
    L = g.dcase.layers[0]
    qv, qs = L.q("mxfp4")
    idx.idx_dense_masked_logits_topk(g.cfg, g.rows, ctx, qv, qs, L.w("bf16"), g.kcaches[0],
                                     g.sched.struct, dout, dout.stride(0), dlog, dlog.stride(0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dout.cpu().numpy(), res["indices"], err_msg="dense != sparse")


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


@pytest.mark.parametrize("q_format", ["mxfp4", "fp8"])
@pytest.mark.parametrize("path", sorted(WEIGHT_PATHS))
def test_nan_scale_bytes_follow_the_nan_rule(path, q_format):
    import dataclasses

    spec = WEIGHT_PATHS[path]
    if q_format == "fp8":
        if path == "rowgroup":
            pytest.skip("row groups serve MXFP4 queries only")
        spec = dataclasses.replace(spec, q_formats=("mxfp4", "fp8"))
    case = _with_nan_inputs(W.generate(spec, seed=19), q_format, seed=23)
    g, res = run_and_compare(case, q_format=q_format, tag=f"nan-{path}-{q_format}")
    # row 1: every logit -inf (its NaN weight), so its lowest tokens win
    ora = oracle.indexer_rows(case, 0, np.array([1], np.int32), q_format)
    assert np.all(ora.row_logits(0) == -np.inf)


def test_fp8_query_products_need_the_bf16_route():
    """Why fp8 queries go through bf16: the MX-scaled fp8 x fp4 MFMA adds its products in a
    narrow adder.  Worked case: 448 + 2^-9 (e4m3 0x7E and 0x01 against e2m1 1.0) comes out
    448 from it, and from the fp8 x fp8 form on K converted exactly to e4m3, and exact from
    the bf16 route.  On random e4m3 / e2m1 data (the workloads' encodings) the logits the
    fp8 x fp4 form gives miss the 1e-5 tolerance, the bf16 route's do not."""
    import sparse_attention_indexer_candidate_amd as idx

    def run(q, kv, ks):
        outs = []
        for mode in (0, 1, 2):
            out = torch.zeros((16, 16), dtype=torch.float32, device=DEV)
            idx.idx_measure_fp8_dot(torch.from_numpy(q).to(DEV), torch.from_numpy(kv).to(DEV),
                                    torch.from_numpy(ks).to(DEV), mode, out)
            outs.append(out)
        torch.cuda.synchronize()
        return [o.cpu().numpy().astype(np.float64) for o in outs]

    def exact(q, kv, ks):
        e4 = np.array([oracle.e4m3fn(b) for b in range(256)])
        e2 = np.array([oracle.e2m1(c) for c in range(16)])
        qd = e4[q]                                                   # [16, 128]
        kd = np.empty((16, 128))
        kd[:, 0::2], kd[:, 1::2] = e2[kv & 15], e2[kv >> 4]
        kd *= np.repeat(np.array([[oracle.ue8m0(int(b)) for b in r] for r in ks]), 32, axis=1)
        terms = qd[:, None, :] * kd[None, :, :]                      # [row, token, d]
        return terms.sum(-1), np.abs(terms).sum(-1)

    q = np.zeros((16, 128), np.uint8)
    kv = np.zeros((16, 64), np.uint8)
    ks = np.full((16, 4), 127, np.uint8)
    q[0, 0], q[0, 1] = 0x7E, 0x01                                    # 448, 2^-9
    kv[0, 0] = 0x22                                                  # elements 0, 1: 1.0
    mx, bf, mx8 = run(q, kv, ks)
    assert mx[0, 0] == 448.0, mx[0, 0]
    assert bf[0, 0] == 448.0 + 2.0 ** -9, bf[0, 0]
    assert mx8[0, 0] != 448.0 + 2.0 ** -9, mx8[0, 0]

    # workload-shaped data: the fp8 query recipe (N(0,1), row scale max/448, e4m3 codes)
    # for 16 heads, e2m1 K of N(0,1) with scales 2^[-4, 4]; 16 heads with U(0,1)/8 weights
    # give each token's logit sum_h w_h ReLU(dot), checked against 1e-6 + 1e-5 |logit|
    rng = np.random.default_rng(7)
    spec = W.Spec(name="acc", num_rows=1, num_heads=16, head_dim=128, q_formats=("fp8",))
    bad = {0: 0, 1: 0, 2: 0}
    worst = {0: 0.0, 1: 0.0, 2: 0.0}
    for trial in range(200):
        q8, rs = W._draw_q_fp8(spec, rng)
        q = np.ascontiguousarray(q8[0])
        kv = W._e2m1_packed(rng, 16 * 128).reshape(16, 64)
        ks = W._ue8m0_scales(rng, (16, 4), (-4, 4))
        want, _ = exact(q, kv, ks)
        w = rng.random(16) / 8.0
        lw = (w[:, None] * np.maximum(want * rs[0], 0.0)).sum(0)
        for mode, got in enumerate(run(q, kv, ks)):
            lg = (w[:, None] * np.maximum(got * rs[0], 0.0)).sum(0)
            err = np.abs(lg - lw)
            bad[mode] += int((err > 1e-6 + 1e-5 * np.abs(lw)).sum())
            worst[mode] = max(worst[mode], float(np.max(err / np.abs(lw))))
    _say(f"[fp8 products] 3200 logits outside the tolerance: MX fp8 x fp4 {bad[0]} (worst "
         f"relative error {worst[0]:.1e}), MX fp8 x fp8 {bad[2]} (worst {worst[2]:.1e}), "
         f"bf16 route {bad[1]} (worst {worst[1]:.1e})")
    assert bad[1] == 0
    assert bad[0] > 0


def test_measurement_kernels_run_and_read_every_word():
    """The roofline's reference kernels: the read stream folds every 32-bit word of its
    buffer into the per-workgroup XORs (checked against numpy), and both MFMA loops give
    finite, repeatable sinks."""
    import sparse_attention_indexer_candidate_amd as idx

    rng = np.random.default_rng(5)
    for nbytes in (1 << 20, (3 << 16) + 48):
        host = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
        src = torch.from_numpy(host.view(np.uint8).copy()).to(DEV)
        sink = torch.zeros(idx.IDX_MEASURE_WGS, dtype=torch.int32, device=DEV)
        idx.idx_measure_read(src, nbytes, sink)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), nbytes
    for fn in (idx.idx_measure_mfma, idx.idx_measure_mfma_relu):
        outs = []
        for _ in range(2):
            sink = torch.full((idx.IDX_MEASURE_WGS * 4,), np.nan, dtype=torch.float32, device=DEV)
            fn(3, sink)
            torch.cuda.synchronize()
            outs.append(sink.cpu().numpy())
        assert np.all(np.isfinite(outs[0])), fn.__name__
        np.testing.assert_array_equal(outs[0], outs[1], err_msg=fn.__name__)

