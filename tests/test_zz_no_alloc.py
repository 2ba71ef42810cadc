"""The entry point that allocates nothing (idx_sparse_mqa_logits_topk_noalloc), through the
C ABI: its indices equal idx_sparse_mqa_logits_topk's (workspace form) bit for bit, on two
calls in a row, the second on a smaller input, on the split plan (its logits live in the
library's static scratch; MXFP4 and fp8 queries) and on the one-row plan (no scratch
needed)."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import GpuRun
from workloads.device import to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _noalloc_matches_workspace_call(case, tag, q_format="mxfp4"):
    import sparse_attention_indexer_candidate_amd as idx

    g = GpuRun(case, to_device(case, DEV), q_format=q_format)
    g.expand()
    print(f"[{tag}] rows={case.num_rows} plan={idx.idx_sparse_plan(g.cfg, case.num_rows)}",
          flush=True)
    g.score(0, with_logits=False)                    # the existing entry point, workspace form
    torch.cuda.synchronize()
    want = g.out.cpu().numpy().copy()
    L = g.dcase.layers[0]
    qv, qs = L.q(q_format)
    out = torch.full_like(g.out, -7)
    idx.idx_sparse_mqa_logits_topk_noalloc(g.cfg, g.rows, qv, qs, L.weights, g.kcaches[0],
                                           g.sched.struct, out, out.stride(0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), want, err_msg=f"{tag}: indices")
    # with logits_out (no scratch): the same logits as the existing call's, bit for bit
    g.score(0, with_logits=True)
    torch.cuda.synchronize()
    ref_logits = g.logits.cpu().numpy().copy()
    lg = torch.empty_like(g.logits)
    out.fill_(-7)
    idx.idx_sparse_mqa_logits_topk_noalloc(g.cfg, g.rows, qv, qs, L.weights, g.kcaches[0],
                                           g.sched.struct, out, out.stride(0), lg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), want, err_msg=f"{tag}: indices (logits_out)")
    np.testing.assert_array_equal(lg.cpu().numpy().view(np.uint32), ref_logits.view(np.uint32),
                                  err_msg=f"{tag}: logits")


def test_noalloc_split_plan_two_calls_second_smaller():
    big = W.generate(W.config(2), 0)                 # 64 rows x 4096 columns: split plan
    small = W.generate(W.Spec(name="na", num_rows=13, page_size=64, cbs=64, nb=20, topk=300,
                              ke_rule="uniform", ke_lo=100, ke_hi=3000, ks_rule="random",
                              cand_rule="messy", fill="all"), seed=3)
    _noalloc_matches_workspace_call(big, "noalloc-split-1")
    _noalloc_matches_workspace_call(small, "noalloc-split-2")


def test_noalloc_split_plan_fp8_queries_two_calls_second_smaller():
    big = W.generate(W.config(5, q_formats=("mxfp4", "fp8")), 0)   # 128 rows: split plan
    small = W.generate(W.Spec(name="nf", num_rows=30, page_size=32, cbs=32, nb=40, topk=200,
                              ke_rule="uniform", ke_lo=100, ke_hi=2000, ks_rule="random",
                              cand_rule="messy", fill="all", q_formats=("mxfp4", "fp8")), seed=6)
    _noalloc_matches_workspace_call(big, "noalloc-fp8-1", "fp8")
    _noalloc_matches_workspace_call(small, "noalloc-fp8-2", "fp8")


def test_noalloc_one_row_plan_two_calls_second_smaller():
    big = W.generate(W.Spec(name="nb", num_rows=300, page_size=64, cbs=64, nb=32, topk=500,
                            ke_rule="uniform", ke_lo=100, ke_hi=4000, cand_rule="messy",
                            fill="all"), seed=4)
    small = W.generate(W.Spec(name="nc", num_rows=260, page_size=64, cbs=64, nb=8, topk=100,
                              ke_rule="uniform", ke_lo=10, ke_hi=900, cand_rule="distinct",
                              fill="all"), seed=5)
    _noalloc_matches_workspace_call(big, "noalloc-rows-1")
    _noalloc_matches_workspace_call(small, "noalloc-rows-2")
