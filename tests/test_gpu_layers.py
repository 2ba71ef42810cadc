"""GPU parity of the multi-layer call: one call against one call per layer bit for bit and
every layer against the oracle, on every launch form, at random shapes and inside replayed
HIP graphs."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import GpuRun, compare_rows
from workloads.device import to_device
from gpu_cases import DEV, THREADS, _check_layers_call, _random_spec, _say

pytestmark = pytest.mark.gpu


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
