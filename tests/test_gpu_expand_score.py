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
from gpu_cases import DEV, THREADS, _say

pytestmark = pytest.mark.gpu


def _spec(name, rows, nb, layers, cbs=64, page=64, topk=300, cand="messy", ks="random"):
    lo, hi = nb * cbs // 3, 2 * nb * cbs
    return W.Spec(name=name, num_rows=rows, page_size=page, cbs=cbs, nb=nb, topk=topk,
                  layers=layers, ke_rule="uniform", ke_lo=lo, ke_hi=hi, ks_rule=ks,
                  cand_rule=cand, fill="all", q_formats=("mxfp4", "fp8"))


# name -> (spec, expansion inside the scoring kernel with MXFP4 queries on a 256-CU device)
CASES = {
    # one layer, fewer than two rows a CU: 1024-thread rows (4 and 8 keys a thread)
    "row_1024_k4": (_spec("es1", 260, 48, 1), True),
    "row_1024_k8": (_spec("es2", 300, 128, 1, topk=2048, cand="distinct", ks="zero"), True),
    # one layer, two rows a CU: 512-thread rows, two a CU (4, 8, 16 keys a thread)
    "row_512_k4": (_spec("es3", 512, 24, 1), True),
    "row_512_k8": (_spec("es4", 512, 64, 1, topk=1000), True),
    "row_512_k16": (_spec("es5", 512, 128, 1, topk=2048), True),
    # several layers, one launch, at most two row-layers a CU: >= CUs rows, or fewer rows
    # but >= CUs row-layers
    "layers_rows": (_spec("es6", 170, 24, 3), True),
    "layers_row_layers": (_spec("es7", 40, 16, 8), True),
    "layers_k8": (_spec("es8", 130, 64, 2, topk=2048), True),
    "layers_k16": (_spec("es9", 256, 128, 2, topk=2048, cand="distinct"), True),
    # more than two rows, or row-layers, a CU: the two launches
    "two_launches_rows": (_spec("es14", 600, 24, 1), False),
    "two_launches_row_layers": (_spec("es15", 300, 24, 3), False),
    # the two launches: 32- and 16-token sparse blocks, fewer
    # row-layers than CUs (split), a prefill chunk's row groups
    "two_launches_nb": (_spec("es10", 260, 160, 2, cbs=32, page=64, topk=1000), False),
    "two_launches_sbk16": (_spec("es11", 260, 40, 2, cbs=16, page=32), False),
    "two_launches_split": (_spec("es12", 40, 30, 2), False),
    "two_launches_groups": (W.Spec(name="es13", num_rows=2050, page_size=128, cbs=64, nb=8,
                                   topk=100, layers=2, mode="prefill", ke_rule="uniform",
                                   ke_lo=1, ke_hi=1500, ks_rule="random", context=1600,
                                   cand_rule="messy", fill="all",
                                   q_formats=("mxfp4", "fp8")), False),
}


def _schedule(g):
    torch.cuda.synchronize()
    return (g.sched.sparse_indices.cpu().numpy().copy(), g.sched.end.cpu().numpy().copy(),
            g.sched.work.cpu().numpy().copy())


def _poison(g):
    g.sched.sparse_indices.fill_(-9)
    g.sched.end.fill_(-9)
    g.sched.work.fill_(0xAB)


def _check(case, tag, q_format, expect_fused=None):
    import sparse_attention_indexer_candidate_amd as idx

    nl = case.spec.layers
    g = GpuRun(case, to_device(case, DEV), q_format=q_format)
    plan = idx.idx_sparse_plan(g.cfg, case.num_rows, nl, logits_home=True)
    if expect_fused is not None and torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert plan["expansion_in_scoring_kernel"] == (expect_fused and q_format == "mxfp4"), plan
    with_logits = [i % 2 == 0 for i in range(nl)]
    _say(f"[{tag}] two calls ({plan['scoring_kernel']})")
    _poison(g)
    g.expand()
    ref_out, ref_log = g.score_layers(range(nl), with_logits)
    ref_sched = _schedule(g)
    _say(f"[{tag}] one call ({plan['expand_and_score_kernel']})")
    _poison(g)
    outs, logs = g.score_layers(range(nl), with_logits, out_pad=3, expand_in_call=True)
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
    spec, fused = CASES[name]
    case = W.generate(spec, seed=31)
    g, outs, logs = _check(case, f"es-{name}-{q_format}", q_format, fused)
    if q_format != "mxfp4":
        return
    # layer 0 against the oracle, from the one call's own schedule and outputs
    res = g.fetch()
    res["indices"] = outs[0].cpu().numpy()
    res["logits"] = logs[0].cpu().numpy()
    ora = oracle.indexer_rows(case, 0, None, q_format, threads=THREADS)
    compare_rows(case, res, ora, case.spec.topk, g.sbk, f"es-{name} layer 0")


@pytest.mark.parametrize("layers", [1, 2])
def test_expand_and_score_drops_pages_outside_the_pool(layers):
    """Table entries outside the pool and table rows outside the tables, expanded inside the
    scoring kernel: the schedule leaves them out as the expansion launch does, and layer 0
    equals the oracle on the clean tables with those blocks removed."""
    spec = dataclasses.replace(_spec("es20", 256, 32, layers), fill="candidates")
    case = W.generate(spec, seed=22)
    bad, clean, bad_rows, _ = corrupt_tables(case, seed=6)
    tag = f"es-drop-l{layers}"
    g, outs, logs = _check(bad, tag, "mxfp4", True)
    si_o, end_o = oracle.expand(clean, g.sbk)
    res = g.fetch()
    np.testing.assert_array_equal(res["sparse_indices"], si_o, err_msg=f"{tag}: schedule")
    np.testing.assert_array_equal(res["end"], end_o, err_msg=f"{tag}: end")
    res["indices"] = outs[0].cpu().numpy()
    res["logits"] = logs[0].cpu().numpy()
    assert np.all(res["indices"][bad_rows] == -1)
    ora = oracle.indexer_rows(clean, 0, None, "mxfp4", threads=THREADS)
    compare_rows(clean, res, ora, spec.topk, g.sbk, tag)


def test_expand_and_score_empty_rows_and_short_candidate_lists():
    """Rows with no candidate at all, or only negative ids, and NB below the two ids a lane
    of the in-kernel expansion (one id a lane)."""
    spec = _spec("es21", 250, 5, 2, topk=200)
    case = W.generate(spec, seed=23)
    case.candidate_blocks[::7] = -1
    case.candidate_blocks[3::11, :2] = -5
    _check(case, "es-empty", "mxfp4", True)
