"""GPU parity of the packed K workspace gather: byte for byte against the oracle, at
random shapes, and scored as a one-page cache."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import GpuRun
from workloads.device import to_device
from gpu_cases import DEV, _say

pytestmark = pytest.mark.gpu


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
