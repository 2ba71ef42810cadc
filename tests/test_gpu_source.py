"""GPU parity of the candidate-source layer (idx_publish_candidates) against the oracle,
through the C ABI, and the two-level pipeline: the published pool feeding a consuming
layer.

Block scores are compared within the fp32 tolerance (a block's score is one of its
tokens' logits); the published blocks follow the near-threshold rule of the token
top-k with blocks in place of tokens; and the publication is exact for the GPU's own
block scores (from its dense logits)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import GpuRun, check_indices, check_logits, compare_rows, corrupt_tables, exact_topk
from workloads.device import to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
THREADS = oracle.default_threads()


def _say(msg):
    print(msg, flush=True)


def publish(case, dcase, layer=0, nb=None, q_format="mxfp4", score_format="fp32", cbs=None):
    """Runs idx_publish_candidates on every row; returns (candidates [R, nb], dense logits
    [R, ctx64]) on the host."""
    import sparse_attention_indexer_candidate_amd as idx

    s = case.spec
    nb = s.nb if nb is None else nb
    cfg = idx.make_config(s.num_heads, s.head_dim,
                          idx.IDX_Q_MXFP4 if q_format == "mxfp4" else idx.IDX_Q_FP8_E4M3_ROWSCALE,
                          s.page_size, s.cbs, 0, nb, min(s.topk, nb * s.cbs),
                          idx.IDX_SCORE_BF16 if score_format == "bf16" else idx.IDX_SCORE_FP32)
    R = case.num_rows
    max_ctx = max(1, int(case.row_ke.max()))
    ctx64 = (max_ctx + 63) // 64 * 64
    rows = idx.make_rows(dcase.row_ke, dcase.row_ks, dcase.row_table)
    L = dcase.layers[layer]
    kc = idx.make_kcache(L.pool, s.page_size, s.head_dim, dcase.block_table)
    cand = torch.full((R, nb + 3), -7, dtype=torch.int32, device=DEV)
    logits = torch.empty((R, ctx64), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(4, idx.idx_publish_workspace_bytes(cfg, R, max_ctx)), dtype=torch.uint8,
                     device=DEV)
    qv, qs = L.q(q_format)
    idx.idx_publish_candidates(cfg, rows, max_ctx, qv, qs, L.w(score_format), kc, cand,
                               cand.stride(0), logits, logits.stride(0), ws, ws.numel())
    # the same call without the logits output publishes the same pool
    cand2 = torch.full_like(cand, -9)
    idx.idx_publish_candidates(cfg, rows, max_ctx, qv, qs, L.w(score_format), kc, cand2,
                               cand2.stride(0), None, 0, ws, ws.numel())
    torch.cuda.synchronize()
    c, c2 = cand.cpu().numpy(), cand2.cpu().numpy()
    np.testing.assert_array_equal(c[:, :nb], c2[:, :nb], err_msg="publication without logits")
    assert np.all(c[:, nb:] == -7), "wrote past the first NB slots"
    return c[:, :nb], logits.cpu().numpy()


def gpu_block_scores(case, r, logits_row):
    """(eligible blocks, their scores) from the GPU's dense logits of row r."""
    s = case.spec
    ks, ke = int(case.row_ks[r]), int(case.row_ke[r])
    if ke <= ks:
        return np.zeros(0, np.int32), np.zeros(0, np.float32)
    blocks = np.arange(ks // s.cbs, (ke - 1) // s.cbs + 1)
    starts = np.maximum(blocks * s.cbs, ks) - ks
    return blocks.astype(np.int32), np.maximum.reduceat(logits_row[ks:ke], starts)


def compare_publication(case, cand, logits, nb, tag, q_format="mxfp4", score_format="fp32",
                        layer=0):
    width = max(1, (int(case.row_ke.max()) + case.spec.cbs - 1) // case.spec.cbs)
    o_cand, o_score = oracle.source_candidates(case, layer, None, nb, q_format, score_format,
                                               threads=THREADS, score_width=width)
    for r in range(case.num_rows):
        what = f"{tag} row {r}"
        gb, gs = gpu_block_scores(case, r, logits[r])
        ob = np.nonzero(~np.isnan(o_score[r]))[0].astype(np.int32)
        os_ = o_score[r, ob]
        np.testing.assert_array_equal(gb, ob, err_msg=f"{what}: eligible blocks")
        # exact for its own block scores
        np.testing.assert_array_equal(cand[r], exact_topk(gb, gs, nb), err_msg=f"{what}: own")
        if score_format == "bf16":
            if np.array_equal(gs.view(np.uint32), os_.astype(np.float32).view(np.uint32)):
                np.testing.assert_array_equal(cand[r], o_cand[r], err_msg=f"{what}: blocks")
            continue
        check_logits(ob, os_, gb, gs, what)
        check_indices(ob, os_, o_cand[r], cand[r], nb, what)


SOURCE_CASES = {
    # cbs 64 (one part a block), ragged contexts, ks > 0
    "cbs64_ks": (W.Spec(name="p1", num_rows=37, page_size=64, cbs=64, nb=16, topk=100,
                        ke_rule="uniform", ke_lo=1, ke_hi=5000, ks_rule="random",
                        cand_rule="distinct", fill="all"), 16),
    # cbs 16 and 32: several blocks a 64-token part group
    "cbs16": (W.Spec(name="p2", num_rows=20, page_size=32, cbs=16, nb=40, topk=50,
                     ke_rule="uniform", ke_lo=10, ke_hi=3000, ks_rule="random",
                     cand_rule="distinct", fill="all"), 40),
    "cbs32": (W.Spec(name="p3", num_rows=20, page_size=64, cbs=32, nb=30, topk=50,
                     ke_rule="uniform", ke_lo=10, ke_hi=3000, cand_rule="distinct",
                     fill="all"), 30),
    # cbs 256: four parts a block; more eligible blocks than NB and fewer
    "cbs256": (W.Spec(name="p4", num_rows=24, page_size=256, cbs=256, nb=8, topk=100,
                      ke_rule="uniform", ke_lo=1, ke_hi=6000, ks_rule="random",
                      cand_rule="distinct", fill="all"), 8),
    # prefill rows on one table
    "prefill": (W.Spec(name="p5", num_rows=300, page_size=64, cbs=64, nb=16, topk=128,
                       mode="prefill", ke_rule="causal", context=300, cand_rule="causal_all",
                       fill="all"), 4),
}


@pytest.mark.parametrize("page_size", [16, 32])
def test_publication_fp8_queries_on_small_pages(page_size):
    """fp8 queries on pages shorter than a 64-token scoring group (tiles resolved one by
    one), every row against the oracle."""
    spec = W.Spec(name=f"pf{page_size}", num_rows=24, page_size=page_size, cbs=page_size, nb=30,
                  topk=100, ke_rule="uniform", ke_lo=10, ke_hi=3000, ks_rule="random",
                  cand_rule="distinct", fill="all", q_formats=("mxfp4", "fp8"))
    case = W.generate(spec, seed=47)
    cand, logits = publish(case, to_device(case, DEV), q_format="fp8")
    compare_publication(case, cand, logits, spec.nb, f"source-fp8-p{page_size}", "fp8")


@pytest.mark.parametrize("name", sorted(SOURCE_CASES))
def test_publication_matches_oracle_all_rows(name):
    spec, nb = SOURCE_CASES[name]
    case = W.generate(spec, seed=41)
    _say(f"[source-{name}] rows={case.num_rows} cbs={spec.cbs} nb={nb}")
    cand, logits = publish(case, to_device(case, DEV), nb=nb)
    compare_publication(case, cand, logits, nb, f"source-{name}")


@pytest.mark.parametrize("i", range(8))
def test_random_publications(i):
    """Seeded random publications: block sizes 16-256 on pages of a multiple of the sparse
    block, NB from 1 to min(64, 8192 / cbs), ragged [ks, ke), both query formats and both
    score formats."""
    rng = np.random.default_rng(9000 + i)
    cbs = int(rng.choice([16, 32, 64, 128, 256]))
    sbk = 64 if cbs % 64 == 0 else cbs
    page_size = int(rng.choice([p for p in (16, 32, 64, 128, 256) if p % sbk == 0]))
    ke_hi = int(rng.integers(cbs, min(4096 * cbs, 20000)))
    nb = int(rng.integers(1, min(64, 8192 // cbs) + 1))   # NB * cbs <= 8192
    spec = W.Spec(name=f"rp{i}", num_rows=int(rng.integers(1, 90)), page_size=page_size, cbs=cbs,
                  nb=nb, topk=min(100, nb * cbs), ke_rule="uniform",
                  ke_lo=int(rng.integers(0, ke_hi)), ke_hi=ke_hi,
                  ks_rule=str(rng.choice(["zero", "random"])), cand_rule="distinct", fill="all",
                  q_formats=("mxfp4", "fp8"))
    q_format = ("mxfp4", "fp8")[i % 2]
    score_format = ("fp32", "bf16")[(i // 2) % 2]
    case = W.generate(spec, seed=90 + i)
    _say(f"[rp{i}] rows={spec.num_rows} cbs={cbs} page={page_size} nb={nb} ke<={ke_hi} "
         f"{q_format} {score_format}")
    cand, logits = publish(case, to_device(case, DEV), q_format=q_format, score_format=score_format)
    compare_publication(case, cand, logits, nb, f"rp{i}", q_format, score_format)


@pytest.mark.parametrize("variant", ["fp8", "bf16", "zero_weights", "signed_weights"])
def test_publication_variants(variant):
    spec = W.Spec(name="pv", num_rows=30, page_size=64, cbs=64, nb=12, topk=100,
                  ke_rule="uniform", ke_lo=100, ke_hi=4000, ks_rule="random",
                  cand_rule="distinct", fill="all", q_formats=("mxfp4", "fp8"))
    case = W.generate(spec, seed=43)
    q_format, score_format = "mxfp4", "fp32"
    if variant == "fp8":
        q_format = "fp8"
    elif variant == "bf16":
        score_format = "bf16"
    else:
        rng = np.random.default_rng(3)
        layers = []
        for L in case.layers:
            w = np.zeros_like(L.weights) if variant == "zero_weights" else \
                ((rng.random(L.weights.shape) * 2 - 1) / 8).astype(np.float32)
            layers.append(dataclasses.replace(L, weights=w))
        case = dataclasses.replace(case, layers=layers)
    _say(f"[source-{variant}]")
    cand, logits = publish(case, to_device(case, DEV), q_format=q_format,
                           score_format=score_format)
    if variant == "zero_weights":
        # every logit +0: every eligible block ties, the lowest NB win
        for r in range(case.num_rows):
            gb, _ = gpu_block_scores(case, r, logits[r])
            want = np.full(12, -1, np.int32)
            want[:min(12, gb.size)] = gb[:12]
            np.testing.assert_array_equal(cand[r], want, err_msg=f"zero weights row {r}")
    if variant == "signed_weights":
        # with signed weights the tolerance's magnitudes come from |w| (as for tokens);
        # the exact-for-own-scores check and the oracle agreement away from ties suffice
        o_cand, _ = oracle.source_candidates(case, 0, None, 12, threads=THREADS)
        agree = np.mean([np.array_equal(cand[r], o_cand[r]) for r in range(case.num_rows)])
        assert agree > 0.9, agree
        for r in range(case.num_rows):
            gb, gs = gpu_block_scores(case, r, logits[r])
            np.testing.assert_array_equal(cand[r], exact_topk(gb, gs, 12))
        return
    compare_publication(case, cand, logits, 12, f"source-{variant}", q_format, score_format)


def test_publication_full_size_comparison_workload():
    """The comparison workload's inputs (128 rows, 64k contexts, every page filled), 64
    blocks of 64 published a row, every row against the oracle."""
    case = W.generate(W.config(5), 0)
    _say("[source-cfg5] publish")
    cand, logits = publish(case, to_device(case, DEV), nb=64)
    compare_publication(case, cand, logits, 64, "source-cfg5")


def test_publication_drops_pages_outside_the_pool_and_invalid_table_rows():
    """The source layer on block-table entries outside the pool and table rows out of range:
    those tokens are not read (-inf logits), a block without a scored token is not eligible,
    a row without a table publishes nothing, every scored token's logit equals bit for bit
    the one the original tables give (that publication checked against the oracle), and the
    publication is exact for the GPU's own block scores."""
    spec = W.Spec(name="pd", num_rows=40, page_size=64, cbs=64, nb=16, topk=200,
                  ke_rule="uniform", ke_lo=300, ke_hi=3000, ks_rule="random",
                  cand_rule="messy", fill="all")
    case = W.generate(spec, seed=21)
    bad, _, bad_rows, bad_pages = corrupt_tables(case, seed=5)
    _say(f"[publish-drop] corrupted entries={int(bad_pages.sum())} bad rows={bad_rows.tolist()}")
    c0, l0 = publish(case, to_device(case, DEV))
    compare_publication(case, c0, l0, spec.nb, "publish-drop original")
    c1, l1 = publish(bad, to_device(bad, DEV))
    ctx = int(case.row_ke.max())
    for r in range(case.num_rows):
        what = f"publish-drop row {r}"
        if r in bad_rows:
            assert np.all(c1[r] == -1) and np.all(l1[r, :ctx] == -np.inf), what
            continue
        ks, ke = int(case.row_ks[r]), int(case.row_ke[r])
        toks = np.arange(ks, ke)
        dropped = bad_pages[case.row_table[r], toks // spec.page_size]
        assert np.all(l1[r, toks[dropped]] == -np.inf), f"{what}: a dropped token was scored"
        np.testing.assert_array_equal(l1[r, toks[~dropped]].view(np.uint32),
                                      l0[r, toks[~dropped]].view(np.uint32), err_msg=what)
        kept = toks[~dropped]
        blocks = np.unique(kept // spec.cbs).astype(np.int32)
        scores = np.array([l1[r, kept[kept // spec.cbs == b]].max() for b in blocks],
                          dtype=np.float32)
        np.testing.assert_array_equal(c1[r], exact_topk(blocks, scores, spec.nb), err_msg=what)


def test_two_level_pipeline_source_then_consumer():
    """Layer 0 publishes each row's pool; the consuming layer 1 expands and scores it.  The
    candidate pool published on the GPU equals the oracle's; the consumer's result on it
    matches the oracle's indexer on the oracle's pool."""
    spec = W.Spec(name="two", num_rows=48, page_size=64, cbs=64, nb=16, topk=300, layers=2,
                  ke_rule="uniform", ke_lo=2000, ke_hi=9000, ks_rule="zero",
                  cand_rule="distinct", fill="all")
    case = W.generate(spec, seed=47)
    dcase = to_device(case, DEV)
    _say("[two-level] publish")
    cand, _ = publish(case, dcase, layer=0)
    o_cand, _ = oracle.source_candidates(case, 0, None, spec.nb, threads=THREADS)
    np.testing.assert_array_equal(cand, o_cand, err_msg="published pools differ")
    consumer = dataclasses.replace(case, candidate_blocks=o_cand)
    dconsumer = dataclasses.replace(dcase, candidate_blocks=torch.from_numpy(cand).to(DEV))
    g = GpuRun(consumer, dconsumer)
    g.expand()
    g.score(1, with_logits=True)
    res = g.fetch()
    ora = oracle.indexer_rows(consumer, 1, threads=THREADS)
    _say("[two-level] consumer")
    compare_rows(consumer, res, ora, spec.topk, g.sbk, "two-level layer 1")
