"""GPU parity at the edges of the inputs: signed and all-zero weights, valid columns whose
logits overflow, pages shorter than a scoring group, [ks, ke) edges and wide strides, pages
and table rows outside the pool, and separate value and scale pools."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import GpuRun, compare_rows, corrupt_tables, exact_topk, gpu_row_tokens
from workloads.device import to_device
from gpu_cases import (
    DEV, DROPPED, THREADS, WEIGHT_PATHS, _dense_indices, _overflowed, _reweighted, _say,
    run_and_compare,
)

pytestmark = pytest.mark.gpu


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
