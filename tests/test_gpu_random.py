"""Seeded random shapes on every launch form and query / score format, and one case for
each kernel instantiation that the other cases leave out, each against the oracle."""

import numpy as np
import pytest

import workloads as W
from gpu_cases import (
    _check_layers_call, _dense_indices, _random_spec, _reweighted, _say, _sweep_spec,
    run_and_compare,
)

pytestmark = pytest.mark.gpu


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
