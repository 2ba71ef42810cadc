"""GPU parity of the HIP path against the CPU oracle, called through the C ABI: the
workloads at full size, small cases across block sizes, ranges and candidate mess, rows of
one request, the bf16 and fp8 variants, NaN inputs, graph replays and the measurement
kernels.  Every row of every case is compared with the oracle (float tolerance and the
near-threshold index rule, and the exact top-k of the GPU's own logits)."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import GpuRun, compare_rows, gpu_row_tokens
from workloads.device import to_device
from gpu_cases import DEV, SMALL, THREADS, WEIGHT_PATHS, _say, _with_nan_inputs, run_and_compare

pytestmark = pytest.mark.gpu


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
    """A step (expansion, sparse scoring, the dense comparator, and the expansion and
    scoring in one call) captured as one HIP graph on its own stream and replayed several
    times, with eager steps of other inputs on the same stream between the replays: every
    replay gives the eager result, bit for bit (the library records no memset and
    allocates nothing)."""
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
            out1 = torch.full((R, s.topk), -7, dtype=torch.int32, device=DEV)
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
                                                       stream=sh),
                     idx.bind_expand_and_score_layers(
                         cfg, rows, d.candidate_blocks, d.candidate_blocks.stride(0),
                         sched.struct, [(qv, qs, d.layers[0].weights, kc, out1, None)],
                         out1.stride(0), ws, ws.numel(), stream=sh)]
            runs.append(dict(keep=(d, rows, kc, sched, ws), calls=calls, out=out, dout=dout,
                             out1=out1))
        for r in runs:                                   # eager results
            for c in r["calls"]:
                c()
        torch.cuda.synchronize()
        for r in runs:
            r["ref"], r["dref"] = r["out"].clone(), r["dout"].clone()
        np.testing.assert_array_equal(runs[0]["ref"].cpu().numpy(), runs[0]["dref"].cpu().numpy())
        for r in runs:
            assert torch.equal(r["out1"], r["ref"]), "one call != expansion + scoring calls"
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in runs[0]["calls"]:
                c()
        other = runs[1]
        for rep in range(3):
            runs[0]["out"].fill_(-7)
            runs[0]["dout"].fill_(-7)
            runs[0]["out1"].fill_(-7)
            other["out"].fill_(-7)
            for c in other["calls"]:                     # eager work between replays
                c()
            g.replay()
            torch.cuda.synchronize()
            _say(f"[graph {which}] replay {rep}")
            assert torch.equal(runs[0]["out"], runs[0]["ref"]), f"replay {rep}: sparse indices"
            assert torch.equal(runs[0]["dout"], runs[0]["dref"]), f"replay {rep}: dense indices"
            assert torch.equal(runs[0]["out1"], runs[0]["ref"]), f"replay {rep}: one call"
            assert torch.equal(other["out"], other["ref"]), f"replay {rep}: eager step"


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
