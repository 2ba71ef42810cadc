"""The GPU parity checker's own rules, on the CPU with synthetic results: the bf16
rounding helper agrees with the oracle's, and planted mistakes in "GPU" results built
from the oracle are caught."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import check_indices_bf16, check_logits_bf16, corrupt_tables, round_bf16_np


def test_round_bf16_np_matches_oracle_rounding():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
                        1.0 + np.arange(-64, 64) * 2.0 ** -9, [0.0, -0.0, 2.0 ** -134,
                                                               3.39617752923046e+38]])
    got = round_bf16_np(x)
    for xi, gi in zip(x, got):
        want = oracle.round_bf16(float(xi))
        assert gi == want and np.signbit(gi) == np.signbit(want), (xi, gi, want)


def _bf16_case():
    spec = W.Spec(name="pr", num_rows=3, num_heads=4, head_dim=64, page_size=16, cbs=16, nb=8,
                  topk=20, ke_rule="uniform", ke_lo=60, ke_hi=128, cand_rule="distinct",
                  fill="all")
    case = W.generate(spec, 2)
    return case, oracle.indexer_rows(case, score_format="bf16")


def test_bf16_checker_accepts_the_oracle_and_allowed_roundings():
    case, ora = _bf16_case()
    for i in range(case.num_rows):
        t, x, o = ora.row_tokens(i), ora.row_exact(i), ora.row_logits(i)
        check_logits_bf16(t, x, o, t, o.copy(), "self")
        check_indices_bf16(t, o, ora.indices[i], o, ora.indices[i], case.spec.topk, "self")


@pytest.mark.parametrize("mistake", ["truncated", "one_ulp_up", "fp32_kept", "index_swap"])
def test_bf16_checker_catches_planted_mistakes(mistake):
    case, ora = _bf16_case()
    caught = False
    for i in range(case.num_rows):
        t, x, o = ora.row_tokens(i), ora.row_exact(i), ora.row_logits(i)
        g, gi = o.copy(), ora.indices[i].copy()
        if mistake == "truncated":       # round toward zero instead of to nearest
            g = (x.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
        elif mistake == "one_ulp_up":
            g = ((o.view(np.uint32) + 0x10000) & 0xFFFF0000).view(np.float32)
        elif mistake == "fp32_kept":     # the fp32 sum not rounded
            g = x.astype(np.float32)
        else:                            # a chosen token swapped for an unchosen one
            out = np.setdiff1d(t, gi)
            if out.size and gi[0] >= 0:
                gi[0] = out[0]
                gi = np.sort(gi)
        try:
            check_logits_bf16(t, x, o, t, g, "m")
            check_indices_bf16(t, o, ora.indices[i], g, gi, case.spec.topk, "m")
        except AssertionError:
            caught = True
    assert caught, mistake


@pytest.mark.parametrize("page_size,mode", [(64, "decode"), (128, "decode"), (64, "prefill")])
def test_corrupted_tables_and_their_clean_candidates(page_size, mode):
    """The inputs of the dropped-page GPU tests: every corrupted block-table entry lies
    outside the pool and was reached by an in-range candidate; the clean candidates are
    the originals minus exactly the blocks on corrupted pages, and nothing for the two rows
    whose table row is out of range."""
    spec = W.Spec(name="ct", num_rows=60, page_size=page_size, cbs=64, nb=12, topk=50, mode=mode,
                  ke_rule="uniform", ke_lo=100, ke_hi=1500, ks_rule="random",
                  context=1600 if mode == "prefill" else 0, cand_rule="messy", fill="all")
    case = W.generate(spec, seed=3)
    bad, clean, bad_rows, bad_pages = corrupt_tables(case, seed=5)
    T, P = case.block_table.shape
    npages = case.layers[0].num_pages
    assert bad_pages.sum() >= 3
    v = bad.block_table[bad_pages].astype(np.int64)
    assert np.all((v < 0) | (v >= npages))
    np.testing.assert_array_equal(bad.block_table[~bad_pages], case.block_table[~bad_pages])
    assert bad.row_table[bad_rows[0]] == -1 and bad.row_table[bad_rows[1]] == T
    np.testing.assert_array_equal(np.delete(bad.row_table, bad_rows),
                                  np.delete(case.row_table, bad_rows))
    np.testing.assert_array_equal(bad.candidate_blocks, case.candidate_blocks)
    reached = np.zeros_like(bad_pages)
    for r in range(case.num_rows):
        c = case.candidate_blocks[r].astype(np.int64)
        c = c[(c >= 0) & (c * spec.cbs < case.row_ke[r])] * spec.cbs // spec.page_size
        reached[case.row_table[r], c[c < P]] = True
    assert np.all(reached[bad_pages])
    for r in range(case.num_rows):
        c, cc = case.candidate_blocks[r], clean.candidate_blocks[r]
        if r in bad_rows:
            assert np.all(cc == -1)
            continue
        for b, bc in zip(c, cc):
            lp = int(b) * spec.cbs // spec.page_size
            on_bad = b >= 0 and lp < P and bad_pages[case.row_table[r], lp]
            assert bc == (-1 if on_bad else b)
