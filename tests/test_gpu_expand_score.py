"""GPU parity of idx_expand_and_score_layers: the expansion and every layer's scoring in
one call give the schedule, indices and logits of idx_expand_candidates followed by
idx_sparse_mqa_logits_topk_layers, bit for bit, on the launches that expand inside the
scoring kernel and on those that keep the two launches; layer 0 is also checked against
the oracle."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import GpuRun, compare_rows, corrupt_tables, padded_tail
from workloads.device import to_device
from gpu_cases import DEV, THREADS, _random_spec, _say

pytestmark = pytest.mark.gpu


def _spec(name, rows, nb, layers, cbs=64, page=64, topk=300, cand="messy", ks="random"):
    lo, hi = nb * cbs // 3, 2 * nb * cbs
    return W.Spec(name=name, num_rows=rows, page_size=page, cbs=cbs, nb=nb, topk=topk,
                  layers=layers, ke_rule="uniform", ke_lo=lo, ke_hi=hi, ks_rule=ks,
                  cand_rule=cand, fill="all", q_formats=("mxfp4", "fp8"))


# name -> (spec, the kernel that streams K in the one call with MXFP4 queries on a 256-CU
# device, workspace for every layer's logits)
CASES = {
    # one layer, fewer than two rows a CU: 1024-thread rows (4 and 8 keys a thread)
    "row_1024_k4": (_spec("es1", 260, 48, 1), "expand_fused_row_kernel", False),
    "row_1024_k8": (_spec("es2", 300, 128, 1, topk=2048, cand="distinct", ks="zero"),
                    "expand_fused_row_kernel", False),
    # one layer, two rows a CU: 512-thread rows, two a CU (4, 8, 16 keys a thread)
    "row_512_k4": (_spec("es3", 512, 24, 1), "expand_fused_row_kernel", False),
    "row_512_k8": (_spec("es4", 512, 64, 1, topk=1000), "expand_fused_row_kernel", False),
    "row_512_k16": (_spec("es5", 512, 128, 1, topk=2048), "expand_fused_row_kernel", False),
    # several layers, one launch, at most two row-layers a CU: >= CUs rows, or fewer rows
    # but >= CUs row-layers
    "layers_rows": (_spec("es6", 170, 24, 3), "expand_fused_layers_kernel", False),
    "layers_row_layers": (_spec("es7", 40, 16, 8), "expand_fused_layers_kernel", False),
    "layers_k8": (_spec("es8", 130, 64, 2, topk=2048), "expand_fused_layers_kernel", False),
    "layers_k16": (_spec("es9", 256, 128, 2, topk=2048, cand="distinct"),
                   "expand_fused_layers_kernel", False),
    # fp8 queries in their 8-wave shapes too: 8192-column layers, short single-layer rows
    "layers_k16_below_two_a_cu": (_spec("es32", 200, 128, 2, topk=2048, cand="distinct"),
                                  "expand_fused_layers_kernel", False),
    "row_short": (_spec("es33", 270, 24, 1), "expand_fused_row_kernel", False),
    # fewer rows (or row-layers) than CUs: the split scoring launch expands (64-, 32- and
    # 16-token sparse blocks), one layer or every layer in one launch pair
    "split_one_layer": (_spec("es16", 64, 64, 1, topk=1000), "score_split_expand_kernel", False),
    "split_one_layer_sbk32": (_spec("es17", 100, 100, 1, cbs=32, page=64),
                              "score_split_expand_kernel", False),
    "split_one_layer_sbk16": (_spec("es19", 30, 120, 1, cbs=16, page=32),
                              "score_split_expand_kernel", False),
    "split_layers": (_spec("es12", 40, 30, 2), "score_split_expand_layers_kernel", True),
    "split_layers_wide": (_spec("es22", 24, 128, 2, topk=7000, cand="distinct"),
                          "score_split_expand_layers_kernel", True),
    "split_layers_sbk32": (_spec("es23", 40, 60, 3, cbs=32, page=64),
                           "score_split_expand_layers_kernel", True),
    # two rows a request (rows_per_request 2: a request's rows placed on one XCD), in the
    # split launch and in the one-row kernel
    "split_rows_per_request": (W.config(6, name="es25", fill="all",
                                        q_formats=("mxfp4", "fp8")),
                               "score_split_expand_kernel", False),
    "row_rows_per_request": (W.config(6, name="es26", num_rows=512, ke_lo=2000, ke_hi=6000,
                                      fill="all", q_formats=("mxfp4", "fp8")),
                             "expand_fused_row_kernel", False),
    # the two launches: more than two row-layers a CU, more than 128 candidate blocks,
    # 16-token sparse blocks in the one-row kernels, split layers without a home for every
    # layer's logits (layer by layer), a prefill chunk's row groups
    "two_launches_rows": (_spec("es14", 600, 24, 1), "fused_row_kernel", False),
    "two_launches_row_layers": (_spec("es15", 300, 24, 3), "fused_layers_kernel", False),
    "two_launches_nb": (_spec("es10", 200, 160, 2, cbs=32, page=64, topk=1000),
                        "fused_layers_kernel", False),
    "two_launches_sbk16": (_spec("es11", 200, 40, 2, cbs=16, page=32), "fused_layers_kernel",
                           False),
    "two_launches_split_no_home": (_spec("es18", 40, 30, 2), "score_split_kernel", False),
    # more split workgroups than are resident at once (200 rows x 16 of 512 columns)
    "two_launches_split_rounds": (_spec("es24", 200, 128, 1, topk=2048, cand="distinct"),
                                  "score_split_kernel", False),
    "two_launches_groups": (W.Spec(name="es13", num_rows=2050, page_size=128, cbs=64, nb=8,
                                   topk=100, layers=2, mode="prefill", ke_rule="uniform",
                                   ke_lo=1, ke_hi=1500, ks_rule="random", context=1600,
                                   cand_rule="messy", fill="all", q_formats=("mxfp4", "fp8")),
                            "row_group_layers_kernel", False),
}


def _schedule(g):
    torch.cuda.synchronize()
    return (g.sched.sparse_indices.cpu().numpy().copy(), g.sched.end.cpu().numpy().copy(),
            g.sched.work.cpu().numpy().copy())


def _poison(g):
    g.sched.sparse_indices.fill_(-9)
    g.sched.end.fill_(-9)
    g.sched.work.fill_(0xAB)


def _check(case, tag, q_format, kernel=None, ws_all=False, cand_pad=0, score_format="fp32"):
    """kernel: the kernel the one call's plan must name with MXFP4 queries on 256 CUs (fp8
    queries: the same kernel where fp8 expands inside, else no expansion inside).
    ws_all: a workspace for every layer's logits.  cand_pad: candidate rows that many ids
    wider than NB (a strided view), the padding holding valid-looking ids."""
    import sparse_attention_indexer_candidate_amd as idx

    nl = case.spec.layers
    g = GpuRun(case, to_device(case, DEV), q_format=q_format, score_format=score_format)
    if cand_pad:
        nb = case.spec.nb
        padded = torch.arange(case.num_rows * (nb + cand_pad), dtype=torch.int32,
                              device=DEV).reshape(case.num_rows, nb + cand_pad) % 7
        padded[:, :nb] = g.dcase.candidate_blocks
        g.dcase.candidate_blocks = padded[:, :nb]
    with_logits = [i % 2 == 0 for i in range(nl)]
    home = all(with_logits) or ws_all
    plan = idx.idx_sparse_plan(g.cfg, case.num_rows, nl, logits_home=home)
    if kernel is not None and torch.cuda.get_device_properties(0).multi_processor_count == 256:
        # fp8 queries expand inside with 64-token sparse blocks only: in the split launches
        # when their workgroups (8 groups of 64 columns each) fit three a CU, in the
        # one-row kernels with fewer than two row-layers a CU (8-wave rows)
        ngroups = -(-case.spec.nb * case.spec.cbs // 64)
        wgs = case.num_rows * nl * -(-ngroups // 8)
        fp8_inside = g.sbk == 64 and (
            (kernel.startswith("score_split_expand") and wgs <= 3 * 256)
            or (kernel.startswith("expand_fused") and case.num_rows * nl < 2 * 256))
        want = kernel if q_format == "mxfp4" or fp8_inside else plan["scoring_kernel"]
        assert plan["expand_and_score_kernel"] == want, plan
    wsl = nl if ws_all else 1
    _say(f"[{tag}] two calls ({plan['scoring_kernel']})")
    _poison(g)
    g.expand()
    ref_out, ref_log = g.score_layers(range(nl), with_logits, workspace_layers=wsl)
    ref_sched = _schedule(g)
    _say(f"[{tag}] one call ({plan['expand_and_score_kernel']})")
    _poison(g)
    outs, logs = g.score_layers(range(nl), with_logits, workspace_layers=wsl, out_pad=3,
                                expand_in_call=True)
    sched = _schedule(g)
    for a, b, what in zip(sched, ref_sched, ("sparse_indices", "end", "work")):
        np.testing.assert_array_equal(a, b, err_msg=f"{tag}: schedule {what}")
    for layer in range(nl):
        np.testing.assert_array_equal(outs[layer].cpu().numpy(), ref_out[layer].cpu().numpy(),
                                      err_msg=f"{tag} layer {layer}: indices")
        assert np.all(padded_tail(outs[layer], 3) == -7), f"{tag} layer {layer}: wrote past k"
        if ref_log[layer] is not None:
            np.testing.assert_array_equal(logs[layer].cpu().numpy().view(np.uint32),
                                          ref_log[layer].cpu().numpy().view(np.uint32),
                                          err_msg=f"{tag} layer {layer}: logits")
    return g, outs, logs


@pytest.mark.parametrize("q_format", ["mxfp4", "fp8"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_expand_and_score_matches_two_calls(name, q_format):
    spec, kernel, ws_all = CASES[name]
    case = W.generate(spec, seed=31)
    g, outs, logs = _check(case, f"es-{name}-{q_format}", q_format, kernel, ws_all)
    if q_format != "mxfp4":
        return
    # layer 0 against the oracle, from the one call's own schedule and outputs
    res = g.fetch()
    res["indices"] = outs[0].cpu().numpy()
    res["logits"] = logs[0].cpu().numpy()
    ora = oracle.indexer_rows(case, 0, None, q_format, threads=THREADS)
    compare_rows(case, res, ora, case.spec.topk, g.sbk, f"es-{name} layer 0")


@pytest.mark.parametrize("rows,layers,kernel", [
    (256, 1, "expand_fused_row_kernel"), (256, 2, "expand_fused_layers_kernel"),
    (64, 1, "score_split_expand_kernel")])
def test_expand_and_score_drops_pages_outside_the_pool(rows, layers, kernel):
    """Table entries outside the pool and table rows outside the tables, expanded inside the
    scoring kernel: the schedule leaves them out as the expansion launch does, and layer 0
    equals the oracle on the clean tables with those blocks removed."""
    spec = dataclasses.replace(_spec("es20", rows, 32, layers), fill="candidates")
    case = W.generate(spec, seed=22)
    bad, clean, bad_rows, _ = corrupt_tables(case, seed=6)
    tag = f"es-drop-r{rows}-l{layers}"
    g, outs, logs = _check(bad, tag, "mxfp4", kernel)
    si_o, end_o = oracle.expand(clean, g.sbk)
    res = g.fetch()
    np.testing.assert_array_equal(res["sparse_indices"], si_o, err_msg=f"{tag}: schedule")
    np.testing.assert_array_equal(res["end"], end_o, err_msg=f"{tag}: end")
    res["indices"] = outs[0].cpu().numpy()
    res["logits"] = logs[0].cpu().numpy()
    assert np.all(res["indices"][bad_rows] == -1)
    ora = oracle.indexer_rows(clean, 0, None, "mxfp4", threads=THREADS)
    compare_rows(clean, res, ora, spec.topk, g.sbk, tag)


@pytest.mark.parametrize("rows,kernel", [(250, "expand_fused_layers_kernel"),
                                         (60, "score_split_expand_layers_kernel")])
def test_expand_and_score_empty_rows_and_short_candidate_lists(rows, kernel):
    """Rows with no candidate at all, or only negative ids, and NB below the two ids a lane
    of the in-kernel expansion (one id a lane)."""
    spec = _spec("es21", rows, 5, 2, topk=200)
    case = W.generate(spec, seed=23)
    case.candidate_blocks[::7] = -1
    case.candidate_blocks[3::11, :2] = -5
    _check(case, f"es-empty-r{rows}", "mxfp4", kernel, ws_all=True)


@pytest.mark.parametrize("rows,layers,kernel", [(64, 1, "score_split_expand_kernel"),
                                                (256, 2, "expand_fused_layers_kernel")])
def test_expand_and_score_wide_candidate_stride(rows, layers, kernel):
    """Candidate rows wider than NB (stride NB + 5) whose padding holds valid-looking ids:
    the one call reads the first NB ids of each row, as the expansion launch does."""
    case = W.generate(_spec("es31", rows, 40, layers), seed=24)
    _check(case, f"es-stride-r{rows}-l{layers}", "mxfp4", kernel, cand_pad=5)


@pytest.mark.parametrize("name", ["split_one_layer", "row_1024_k4", "layers_row_layers"])
def test_expand_and_score_bf16_scoring(name):
    """bf16 weights and bf16-rounded logits through the one call (split, one-row and
    multi-layer forms): the same schedule, indices and logits as the two calls, and layer 0
    against the oracle's bf16 scoring."""
    spec, kernel, ws_all = CASES[name]
    case = W.generate(spec, seed=33)
    g, outs, logs = _check(case, f"es-bf16-{name}", "mxfp4", kernel, ws_all,
                           score_format="bf16")
    res = g.fetch()
    res["indices"] = outs[0].cpu().numpy()
    res["logits"] = logs[0].cpu().numpy()
    ora = oracle.indexer_rows(case, 0, None, "mxfp4", threads=THREADS, score_format="bf16")
    compare_rows(case, res, ora, case.spec.topk, g.sbk, f"es-bf16-{name} layer 0",
                 score_format="bf16")


@pytest.mark.parametrize("i", range(12))
def test_random_expand_and_score_calls(i):
    """Seeded random one calls against the two calls, bit for bit: 1-8 layers, row counts
    that take each placement (split launches, one-row kernels in one round, more rounds,
    row groups), random block and page sizes, k, ranges and candidate mess, both query
    formats; the plan names no expectation here (the fixed cases pin it)."""
    rng = np.random.default_rng(9000 + i)
    spec, _ = _random_spec(400 + i)
    layers = int(rng.integers(1, 9))
    form = i % 4
    rows = [int(rng.integers(4, 120)), int(rng.integers(256 // layers + 1, 2 * 256 // layers)),
            int(rng.integers(256, 420)), spec.num_rows][form]
    if form == 3 and spec.mode != "prefill":
        spec = dataclasses.replace(spec, mode="prefill", ke_lo=1, context=spec.ke_hi)
        rows = 2048 + int(rng.integers(0, 40))
    spec = dataclasses.replace(spec, name=f"re{i}", num_rows=max(rows, 1), layers=layers,
                               q_formats=("mxfp4", "fp8"))
    q_format = ("mxfp4", "fp8")[(i + i // 4) % 2]
    _say(f"[re{i}] rows={spec.num_rows} layers={layers} cbs={spec.cbs} page={spec.page_size} "
         f"nb={spec.nb} k={spec.topk} {spec.mode} {q_format}")
    _check(W.generate(spec, seed=90 + i), f"re{i}", q_format, ws_all=bool(i % 2))
