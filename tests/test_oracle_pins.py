"""Pins of the CPU oracle against things other than itself (CPU only).

* element decodes against hand-derived tables and PyTorch's fp8 / e8m0 decodes;
* closed-form logits (constant inputs, flipped heads, one-hot scale blocks,
  the fp8-Q variant) whose values follow by hand from the definition;
* a textbook special case (one head, unit weight, unit scales) that reduces to
  an integer dot product and numpy's lexsort;
* the independent dense-then-mask brute force on hundreds of tiny random cases;
* invariants of the output and arithmetic-free special cases (k >= valid count,
  all-equal logits).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from brute_force import row as brute_row
from brute_force import source_row as brute_source_row
from golden_io import bf16_examples, e2m1_table, packed_examples, scale_fp8_examples

pytestmark = []


# ---------------------------------------------------------------- decodes ----

def test_e2m1_matches_hand_table():
    table = e2m1_table()
    for code, v in table.items():
        got = oracle.e2m1(code)
        assert got == v and np.signbit(got) == np.signbit(v), (hex(code), got, v)


def test_ue8m0_matches_torch_e8m0():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64)
    for b in range(255):
        assert oracle.ue8m0(b) == ref[b].item(), b
    assert np.isnan(oracle.ue8m0(255)) and torch.isnan(ref[255])


def test_e4m3fn_matches_torch_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for b in range(256):
        got, want = oracle.e4m3fn(b), ref[b].item()
        if np.isnan(want):
            assert np.isnan(got), hex(b)
        else:
            assert got == want and np.signbit(got) == np.signbit(want), (hex(b), got, want)


def test_hand_worked_scale_and_fp8_examples():
    for kind, b, v in scale_fp8_examples():
        got = oracle.ue8m0(b) if kind == "ue8m0" else oracle.e4m3fn(b)
        assert got == v and np.signbit(got) == np.signbit(v), (kind, b, got, v)


def test_bf16_decode_matches_torch_bfloat16():
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    for c in range(65536):
        got, want = oracle.bf16(c), ref[c]
        if np.isnan(want):
            assert np.isnan(got), hex(c)
        else:
            assert got == want and np.signbit(got) == np.signbit(want), (hex(c), got, want)


def test_bf16_hand_worked_roundings_and_decodes():
    for kind, x, want in bf16_examples():
        got = oracle.round_bf16(x) if kind == "round" else oracle.bf16(x)
        assert got == want and np.signbit(got) == np.signbit(want), (kind, x, got, want)


def test_bf16_rounding_matches_torch_on_fp32_values():
    """For binary32 inputs one rounding to bf16 is PyTorch's float -> bfloat16 conversion
    (round to nearest even); the bit patterns cover every binade, subnormals and both
    signs, plus the halfway cases of each (low 16 bits 0x8000)."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    halfway = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    bits = np.concatenate([bits, halfway])
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    for xi, want in zip(x, ref):
        got = oracle.round_bf16(float(xi))
        assert got == want and np.signbit(got) == np.signbit(want), (float(xi), got, want)


def test_bf16_scoring_closed_form_ties_after_rounding():
    # One head, weight 1 (bf16 0x3F80), Q scales 2^0.  Q: element 0 = 4.0 (code 6), block
    # 1 all 1.0 (code 2).  K of token t: element 0 = 4.0 with block scale 2^6 (4 * 4 * 64
    # = 1024), the first t elements of block 1 = 1.0 with block scale 2^2 (+ 4t):
    # dot_t = 1024 + 4t.  fp32 logits are all distinct: top-4 = {12, 13, 14, 15}.  In bf16
    # the spacing is 8 on [1024, 2048), so 1024 + 4t rounds to (by hand, ties to even):
    want_bf16 = [1024, 1032, 1032, 1040, 1040, 1040, 1048, 1056,
                 1056, 1056, 1064, 1072, 1072, 1072, 1080, 1088]
    # except token 1, which also gets 2^-14 from block 2 (Q 1.0 against K 0.5 * 2^-13):
    # its exact logit 1028 + 2^-14 lies just above the bf16 tie 1028 and rounds to 1032,
    # while its fp32 logit is 1028 (2^-14 is half of fp32's spacing there, a tie to the
    # even 1028), which a second rounding would send to 1024.
    # top-4 in bf16: 1088 (t=15), 1080 (14), then the three-way tie at 1072 (11, 12, 13)
    # gives the two lower tokens 11 and 12.
    case = _one_row_case(H=1, D=128, topk=4)
    L = case.layers[0]
    L.weights[:] = 1.0
    qv = np.zeros(64, np.uint8)
    qv[0] = 0x06
    qv[16:32] = 0x22
    qv[32] = 0x02                                        # element 64 (block 2): 1.0
    L.q_values[0, 0] = qv
    for t in range(16):
        kv = np.zeros(64, np.uint8)
        kv[0] = 0x06
        for d in range(32, 32 + t):
            kv[d // 2] |= 0x2 << (4 * (d & 1))
        if t == 1:
            kv[32] = 0x01                                # element 64: 0.5, block scale 2^-13
        _set_k(case, t, kv, np.array([127 + 6, 127 + 2, 127 - 13, 127], np.uint8))
    res = oracle.indexer_rows(case)
    np.testing.assert_array_equal(res.row_logits(0), 1024.0 + 4.0 * np.arange(16))
    np.testing.assert_array_equal(res.indices[0], [12, 13, 14, 15])
    resb = oracle.indexer_rows(case, score_format="bf16")
    np.testing.assert_array_equal(resb.row_logits(0), np.array(want_bf16, np.float32))
    np.testing.assert_array_equal(resb.indices[0], [11, 12, 14, 15])


@pytest.mark.parametrize("chunk", range(4))
def test_bf16_scoring_matches_brute_force(chunk):
    """bf16 weights and bf16-rounded logits: the oracle against the dense-then-mask brute
    force, whose rounding is exact rational arithmetic and whose weight decode is
    PyTorch's."""
    for i in range(chunk * 25, chunk * 25 + 25):
        rng = np.random.default_rng(5000 + i)
        spec = _tiny_spec(rng, i)
        case = W.generate(spec, seed=100 + i)
        pool = case.layers[0].host_pool(spec.page_bytes)
        res = oracle.indexer_rows(case, pool=pool, score_format="bf16")
        for r in range(case.num_rows):
            idx, toks, lg = brute_row(case, r, pool=pool, score_format="bf16")
            np.testing.assert_array_equal(res.row_tokens(r), toks, err_msg=f"case {i} row {r}")
            np.testing.assert_array_equal(res.row_logits(r), lg, err_msg=f"case {i} row {r}")
            np.testing.assert_array_equal(res.indices[r], idx, err_msg=f"case {i} row {r}")


# ------------------------------------------------------ hand-built cases ----

def _one_row_case(H, D, ps=16, n_tokens=16, cbs=16, nb=1, topk=4, q_format="mxfp4"):
    """A one-row decode case with every array set explicitly by the caller."""
    spec = W.Spec(name="hand", num_rows=1, num_heads=H, head_dim=D, page_size=ps, cbs=cbs,
                  nb=nb, topk=topk, q_formats=(q_format,))
    n_pages = (n_tokens + ps - 1) // ps
    L = W.LayerData(weights=np.zeros((1, H), np.float32), num_pages=n_pages + 2,
                    filled_pages=np.arange(n_pages, dtype=np.int64) + 2,
                    filled_data=np.zeros((n_pages, spec.page_bytes), np.uint8))
    if q_format == "mxfp4":
        L.q_values = np.zeros((1, H, D // 2), np.uint8)
        L.q_scales = np.full((1, H, D // 32), 127, np.uint8)
    else:
        L.q_fp8 = np.zeros((1, H, D), np.uint8)
        L.q_rowscale = np.ones(1, np.float32)
    table = np.full((1, n_pages), -1, np.int32)
    table[0] = np.arange(n_pages) + 2           # logical page p -> physical page p + 2
    case = W.Case(spec=spec, seed=0, row_ks=np.zeros(1, np.int32),
                  row_ke=np.array([n_tokens], np.int32), row_table=np.zeros(1, np.int32),
                  block_table=table,
                  candidate_blocks=np.arange(nb, dtype=np.int32)[None, :].copy(), layers=[L])
    return case


def _set_k(case, t, values_bytes, scale_bytes):
    s = case.spec
    L = case.layers[0]
    page = t // s.page_size - 0   # logical page; filled_data row = logical page
    j = t % s.page_size
    D = s.head_dim
    L.filled_data[page, j * (D // 2):(j + 1) * (D // 2)] = values_bytes
    off = s.values_bytes + j * (D // 32)
    L.filled_data[page, off:off + D // 32] = scale_bytes


def test_closed_form_constant_inputs_give_1024():
    # Q elements 1.0 (bytes 0x22, scale 2^0); K elements 0.5 (bytes 0x11, scale 2^1):
    # every term is 1.0 * 0.5 * 2 = 1, every dot 128, logit = 64 * (1/8) * 128 = 1024.
    case = _one_row_case(H=64, D=128, topk=16)
    L = case.layers[0]
    L.q_values[:] = 0x22
    L.weights[:] = 1.0 / 8.0
    for t in range(16):
        _set_k(case, t, 0x11, 128)
    res = oracle.indexer_rows(case)
    assert res.count[0] == 16
    assert np.all(res.row_logits(0) == 1024.0)
    assert list(res.indices[0]) == list(range(16))
    # Flipping head h's Q to -1.0 (0xAA) makes its dot -128, which ReLU removes:
    # each flipped head takes away exactly (1/8) * 128 = 16.
    for nflip in (1, 5, 64):
        L.q_values[0, :nflip] = 0xAA
        res = oracle.indexer_rows(case)
        assert np.all(res.row_logits(0) == 1024.0 - 16.0 * nflip), nflip
        L.q_values[:] = 0x22


def test_nan_rules():
    # UE8M0 0xFF is NaN: a token whose K scale block is NaN has a NaN dot on every head,
    # ReLU maps each to 0, so its logit is 0; a NaN Q scale block on head 5 removes that
    # head from every token (1024 - 16 = 1008 with the constant inputs below).  A NaN
    # weight makes every logit NaN, which ranks as -inf: the lowest tokens win.
    case = _one_row_case(H=64, D=128, topk=16)
    L = case.layers[0]
    L.q_values[:] = 0x22
    L.weights[:] = 1.0 / 8.0
    for t in range(16):
        _set_k(case, t, 0x11, np.array([128, 255 if t in (3, 9) else 128, 128, 128], np.uint8))
    res = oracle.indexer_rows(case)
    want = np.full(16, 1024.0, np.float32)
    want[[3, 9]] = 0.0
    np.testing.assert_array_equal(res.row_logits(0), want)
    case.spec = W.Spec(**{**case.spec.__dict__, "topk": 14})
    res = oracle.indexer_rows(case)
    np.testing.assert_array_equal(res.indices[0], [t for t in range(16) if t not in (3, 9)])
    L.q_scales[0, 5, 2] = 255
    res = oracle.indexer_rows(case)
    want[[t for t in range(16) if t not in (3, 9)]] = 1008.0
    np.testing.assert_array_equal(res.row_logits(0), want)
    L.weights[0, 11] = np.nan
    res = oracle.indexer_rows(case)
    assert np.all(res.row_logits(0) == -np.inf)
    np.testing.assert_array_equal(res.indices[0], list(range(14)))


def test_closed_form_weights_are_per_head():
    # Only head 3 is positive: logit = w[3] * 128 whatever the other weights are.
    case = _one_row_case(H=8, D=128, topk=16)
    L = case.layers[0]
    L.q_values[:] = 0xAA
    L.q_values[0, 3] = 0x22
    L.weights[0] = np.arange(8, dtype=np.float32) + 1.0
    for t in range(16):
        _set_k(case, t, 0x11, 128)
    res = oracle.indexer_rows(case)
    assert np.all(res.row_logits(0) == 4.0 * 128.0)


@pytest.mark.parametrize("d0", list(range(0, 128, 1)))
def test_one_hot_element_and_scale_block(d0):
    # Q: element d0 = 1.0 with its block scale 2^e1; K of token t: element d0 = code
    # c_t with its block scale 2^e2.  dot = e2m1(c_t) * 2^(e1 + e2), logit = ReLU(dot).
    D = 128
    case = _one_row_case(H=1, D=D, topk=16)
    L = case.layers[0]
    L.weights[:] = 1.0
    e1 = (d0 % 7) - 3
    qv = np.zeros(D // 2, np.uint8)
    qv[d0 // 2] = (0x2 << 4) if d0 & 1 else 0x2
    L.q_values[0, 0] = qv
    L.q_scales[0, 0] = 127
    L.q_scales[0, 0, d0 // 32] = 127 + e1
    table = e2m1_table()
    expect = []
    for t in range(16):
        c = t                       # codes 0..15 over the 16 tokens
        e2 = (t % 5) - 2
        kv = np.full(D // 2, 0x77, np.uint8)          # every other element is 6.0 ...
        kv[d0 // 2] = (c << 4) | 0x7 if d0 & 1 else (0x70 | c)
        ks = np.full(D // 32, 127, np.uint8)
        ks[d0 // 32] = 127 + e2
        _set_k(case, t, kv, ks)
        expect.append(max(table[c] * 2.0 ** (e1 + e2), 0.0))
    # ... but Q is zero there, so only element d0 contributes.
    res = oracle.indexer_rows(case)
    np.testing.assert_array_equal(res.row_logits(0), np.array(expect, np.float32))


def test_closed_form_fp8_q_with_row_scale():
    # Q e4m3 1.0 (0x38) everywhere with row scale 0.5; K 0.5 with scale 2^1:
    # dot = 128 * 1.0 * 1.0 = 128, times 0.5 = 64; logit = 64 heads * (1/8) * 64 = 512.
    case = _one_row_case(H=64, D=128, topk=16, q_format="fp8")
    L = case.layers[0]
    L.q_fp8[:] = 0x38
    L.q_rowscale[:] = 0.5
    L.weights[:] = 1.0 / 8.0
    for t in range(16):
        _set_k(case, t, 0x11, 128)
    res = oracle.indexer_rows(case, q_format="fp8")
    assert np.all(res.row_logits(0) == 512.0)
    # Negative row direction: Q -1.0 (0xB8) makes every dot negative -> all logits 0.
    L.q_fp8[:] = 0xB8
    res = oracle.indexer_rows(case, q_format="fp8")
    assert np.all(res.row_logits(0) == 0.0)


def test_packed_nibble_order_examples():
    # Each golden byte as K element pair (0, 1) against one-hot Q picks its halves.
    for byte, e0, e1 in packed_examples():
        for d0, want in ((0, e0), (1, e1)):
            case = _one_row_case(H=1, D=32, topk=1, n_tokens=16, cbs=16)
            L = case.layers[0]
            L.weights[:] = 1.0
            qv = np.zeros(16, np.uint8)
            qv[0] = 0x2 << 4 if d0 else 0x2        # Q element d0 = 1.0
            L.q_values[0, 0] = qv
            kv = np.zeros(16, np.uint8)
            kv[0] = byte
            _set_k(case, 0, kv, 127)
            res = oracle.indexer_rows(case)
            assert res.row_logits(0)[0] == max(want, 0.0), (hex(byte), d0)


# ------------------------------------------------------ textbook case -------

@pytest.mark.parametrize("seed", range(20))
def test_textbook_single_head_integer_dot(seed):
    # H = 1, w = 1, all scales 2^0: logit = ReLU(sum_d q_d k_d) with e2m1 values, i.e.
    # an integer dot product of doubled codes divided by 4; top-k = lexsort.
    spec = W.Spec(name="tb", num_rows=2, num_heads=1, head_dim=64, page_size=8, cbs=8, nb=6,
                  topk=9, ke_rule="uniform", ke_lo=20, ke_hi=60, scale_exp=(0, 0),
                  cand_rule="messy", fill="all")
    case = W.generate(spec, seed)
    L = case.layers[0]
    L.weights[:] = 1.0
    twice = np.array([int(round(2 * e2m1_table()[c])) for c in range(16)], np.int64)
    pool = L.host_pool(spec.page_bytes)
    res = oracle.indexer_rows(case, pool=pool)
    q2 = np.empty(64, np.int64)
    for r in range(case.num_rows):
        q2[0::2] = twice[L.q_values[r, 0] & 15]
        q2[1::2] = twice[L.q_values[r, 0] >> 4]
        toks = res.row_tokens(r)
        want = []
        for t in toks:
            page = case.block_table[case.row_table[r], t // 8]
            vals = pool[page, (t % 8) * 32:(t % 8 + 1) * 32]
            k2 = np.empty(64, np.int64)
            k2[0::2] = twice[vals & 15]
            k2[1::2] = twice[vals >> 4]
            want.append(max(int(q2 @ k2), 0) / 4.0)
        want = np.array(want, np.float32)
        np.testing.assert_array_equal(res.row_logits(r), want)
        order = np.lexsort((toks, -want.astype(np.float64)))
        count = min(spec.topk, toks.size)
        exp = np.full(spec.topk, -1, np.int32)
        exp[:count] = np.sort(toks[order[:count]])
        np.testing.assert_array_equal(res.indices[r], exp)


# ------------------------------------------------------ brute force ---------

def _tiny_spec(rng, i):
    H = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([32, 64, 128]))
    ps = int(rng.choice([4, 8, 16]))
    cbs = int(rng.choice([8, 16]))
    mode = "prefill" if i % 4 == 3 else "decode"
    R = int(rng.integers(1, 5))
    ke_lo = int(rng.integers(1, 150))
    ke_hi = int(rng.integers(ke_lo, 300))
    return W.Spec(name=f"tiny{i}", num_rows=R, num_heads=H, head_dim=D, page_size=ps, cbs=cbs,
                  nb=int(rng.integers(1, 12)), topk=int(rng.integers(1, 64)),
                  mode=mode, ke_rule="uniform", ke_lo=ke_lo, ke_hi=ke_hi,
                  context=ke_hi, ks_rule="random" if i % 3 else "zero",
                  cand_rule=["messy", "distinct"][i % 2], fill="all",
                  q_formats=("mxfp4", "fp8") if i % 5 == 0 else ("mxfp4",))


@pytest.mark.parametrize("chunk", range(10))
def test_oracle_matches_dense_then_mask_brute_force(chunk):
    for i in range(chunk * 30, chunk * 30 + 30):
        rng = np.random.default_rng(1000 + i)
        spec = _tiny_spec(rng, i)
        case = W.generate(spec, seed=i)
        pool = case.layers[0].host_pool(spec.page_bytes)
        for fmt in spec.q_formats:
            res = oracle.indexer_rows(case, pool=pool, q_format=fmt)
            for r in range(case.num_rows):
                idx, toks, lg = brute_row(case, r, q_format=fmt, pool=pool)
                np.testing.assert_array_equal(res.row_tokens(r), toks, err_msg=f"case {i} row {r}")
                np.testing.assert_array_equal(res.row_logits(r), lg, err_msg=f"case {i} row {r}")
                np.testing.assert_array_equal(res.indices[r], idx, err_msg=f"case {i} row {r}")


def test_oracle_matches_brute_force_on_one_page_workspace():
    """A prefill chunk's K packed into one page that holds every position of the
    request (the contiguous K-workspace form of the prefill path on the backend
    page): one block-table entry, token t at slot t of page 0."""
    for seed in range(3):
        spec = W.Spec(name=f"onepage{seed}", num_rows=20, num_heads=4, head_dim=64, page_size=256,
                      cbs=16, nb=10, topk=30, mode="prefill", ke_rule="uniform", ke_lo=1, ke_hi=256,
                      ks_rule="random", context=256, cand_rule="messy", fill="all")
        case = W.generate(spec, seed=seed)
        assert case.block_table.shape == (1, 1)
        pool = case.layers[0].host_pool(spec.page_bytes)
        res = oracle.indexer_rows(case, pool=pool)
        for r in range(case.num_rows):
            idx, toks, lg = brute_row(case, r, pool=pool)
            np.testing.assert_array_equal(res.row_tokens(r), toks, err_msg=f"seed {seed} row {r}")
            np.testing.assert_array_equal(res.row_logits(r), lg, err_msg=f"seed {seed} row {r}")
            np.testing.assert_array_equal(res.indices[r], idx, err_msg=f"seed {seed} row {r}")


def test_workspace_gather_hand_worked():
    """Two requests over three pages of two positions (D = 128: 64 value bytes and 4
    scale bytes a position); request 1's second logical page is out of range."""
    ps, D = 2, 128
    pool = np.zeros((3, ps * 68), np.uint8)
    V = lambda pg, slot: (np.arange(64) + 50 * pg + 7 * slot) % 256
    S = lambda pg, slot: np.array([200 + 3 * pg + slot, pg, slot, 9])
    for pg in range(3):
        for slot in range(ps):
            pool[pg, slot * 64:(slot + 1) * 64] = V(pg, slot)
            pool[pg, ps * 64 + slot * 4:ps * 64 + slot * 4 + 4] = S(pg, slot)
    bt = np.array([[2, 0], [1, 5]], np.int32)       # page 5 does not exist
    cu = [0, 3, 6]                                   # request 0: 3 positions, request 1: 3
    vals, scs = oracle.gather_k_workspace(pool, ps, D, bt, cu, max_tokens=7, fill=0xAB)
    want = [(2, 0), (2, 1), (0, 0), (1, 0), (1, 1)]  # (page, slot) of rows 0..4 by hand
    for row, (pg, slot) in enumerate(want):
        np.testing.assert_array_equal(vals[row], V(pg, slot), err_msg=f"row {row}")
        np.testing.assert_array_equal(scs[row], S(pg, slot), err_msg=f"row {row}")
    assert np.all(vals[5] == 0) and np.all(scs[5] == 0)        # out-of-range page: zeros
    assert np.all(vals[6] == 0xAB) and np.all(scs[6] == 0xAB)  # never written
    # request table, length cap and row cap
    vals, scs = oracle.gather_k_workspace(pool, ps, D, bt, cu, req_table=[1, 0], max_seq_len=2,
                                          max_tokens=4, fill=0xAB)
    for row, (pg, slot) in enumerate([(1, 0), (1, 1), (0xAB, None), (2, 0)]):
        if slot is None:
            assert np.all(vals[row] == 0xAB)                   # p = 2 >= max_seq_len
        else:
            np.testing.assert_array_equal(vals[row], V(pg, slot), err_msg=f"row {row}")


def test_oracle_on_gathered_workspace_equals_paged_cache():
    """Scoring a chunk from its gathered workspace (one page holding every position) gives
    the paged cache's logits and indices exactly: the gather moves bytes only."""
    import dataclasses

    for seed in range(2):
        spec = W.Spec(name=f"ws{seed}", num_rows=24, num_heads=4, head_dim=64, page_size=32,
                      cbs=16, nb=10, topk=30, mode="prefill", ke_rule="uniform", ke_lo=1,
                      ke_hi=320, ks_rule="random", context=320, cand_rule="messy", fill="all")
        case = W.generate(spec, seed=seed)
        pool = case.layers[0].host_pool(spec.page_bytes)
        paged = oracle.indexer_rows(case, pool=pool)
        n = 320
        vals, scs = oracle.gather_k_workspace(pool, spec.page_size, spec.head_dim,
                                              case.block_table, [0, n], req_table=[0])
        ws_spec = dataclasses.replace(spec, page_size=n)
        ws_case = dataclasses.replace(case, spec=ws_spec, block_table=np.zeros((1, 1), np.int32))
        ws_pool = np.concatenate([vals.ravel(), scs.ravel()])[None, :]
        assert ws_pool.shape[1] == ws_spec.page_bytes
        packed = oracle.indexer_rows(ws_case, pool=ws_pool)
        np.testing.assert_array_equal(packed.indices, paged.indices)
        np.testing.assert_array_equal(packed.count, paged.count)
        for i in range(case.num_rows):
            np.testing.assert_array_equal(packed.row_tokens(i), paged.row_tokens(i))
            np.testing.assert_array_equal(packed.row_logits(i).view(np.uint32),
                                          paged.row_logits(i).view(np.uint32))


# ------------------------------------------------------ invariants -----------

def _check_invariants(case, res):
    s = case.spec
    for i, r in enumerate(res.rows):
        ks, ke = int(case.row_ks[r]), int(case.row_ke[r])
        blocks = set(int(b) for b in case.candidate_blocks[r] if b >= 0)
        valid = sum(1 for b in blocks for t in range(b * s.cbs, (b + 1) * s.cbs) if ks <= t < ke)
        count = min(s.topk, valid)
        out = res.indices[i]
        assert res.count[i] == valid
        assert np.all(out[count:] == -1)
        chosen = out[:count]
        assert np.all(chosen >= ks) and np.all(chosen < ke)
        assert all(int(t) // s.cbs in blocks for t in chosen)
        assert np.all(np.diff(chosen) > 0)             # unique, ascending
        # every chosen logit >= every unchosen one; ties resolved toward lower t
        toks, lg = res.row_tokens(i), res.row_logits(i)
        sel = np.isin(toks, chosen)
        if count and (~sel).any():
            lo = lg[sel].min()
            hi = lg[~sel].max()
            assert lo >= hi
            if lo == hi:
                assert toks[sel & (lg == lo)].max() < toks[~sel & (lg == hi)].min()


@pytest.mark.parametrize("n", [1, 2])
def test_invariants_on_workload_shapes(n):
    case = W.generate(W.config(n), 0)
    rows = np.arange(min(8, case.num_rows), dtype=np.int32)
    res = oracle.indexer_rows(case, rows=rows)
    _check_invariants(case, res)


def test_invariants_on_messy_cases():
    for i in range(40):
        spec = W.Spec(name="m", num_rows=3, num_heads=4, head_dim=32, page_size=8, cbs=8, nb=10,
                      topk=int(1 + i % 40), ke_rule="uniform", ke_lo=1, ke_hi=200,
                      ks_rule="random", cand_rule="messy", fill="all")
        case = W.generate(spec, i)
        _check_invariants(case, oracle.indexer_rows(case))


def test_k_at_least_valid_count_returns_all_valid_tokens():
    # Causal prefill rows with i + 1 <= topk: the answer is 0..i then -1, whatever
    # the logits are.
    spec = W.Spec(name="c", num_rows=200, num_heads=2, head_dim=32, page_size=16, cbs=16,
                  nb=16, topk=128, mode="prefill", ke_rule="causal", context=256,
                  cand_rule="causal_all", fill="all")
    case = W.generate(spec, 3)
    res = oracle.indexer_rows(case)
    for i in range(128):
        want = np.full(128, -1, np.int32)
        want[:i + 1] = np.arange(i + 1)
        np.testing.assert_array_equal(res.indices[i], want)


def test_all_equal_logits_take_lowest_tokens():
    # K all zero -> every logit is 0 -> ties everywhere -> the lowest tokens win.
    spec = W.Spec(name="z", num_rows=2, num_heads=2, head_dim=32, page_size=8, cbs=8, nb=5,
                  topk=13, ke_rule="fixed", ke_lo=64, ke_hi=64, fill="all")
    case = W.generate(spec, 1)
    case.layers[0].filled_data[:] = 0
    res = oracle.indexer_rows(case)
    for i in range(2):
        toks = res.row_tokens(i)
        assert np.all(res.row_logits(i) == 0)
        np.testing.assert_array_equal(res.indices[i], np.sort(toks)[:13])


# ------------------------------------------------------ schedule -------------

def test_expand_matches_token_set_definition():
    for i in range(300):
        rng = np.random.default_rng(i)
        cbs = int(rng.choice([16, 32, 64, 128]))
        sbk = int(rng.choice([s for s in (16, 32, 64) if cbs % s == 0]))
        nb = int(rng.integers(1, 20))
        ke = int(rng.integers(0, 3000))
        ks = int(rng.integers(0, ke + 1)) if i % 2 else 0
        cand = rng.integers(-3, (ke + cbs - 1) // cbs + 3, size=nb).astype(np.int32)
        nsb = nb * (cbs // sbk)
        si, n, end = oracle.expand_row(cand, cbs, sbk, ks, ke, nsb)
        toks = set(t for b in set(int(x) for x in cand if x >= 0)
                   for t in range(b * cbs, (b + 1) * cbs) if ks <= t < ke)
        want = sorted(set(t // sbk for t in toks))
        assert end == len(toks)
        assert n == len(want)
        np.testing.assert_array_equal(si[:n], want)
        assert np.all(si[n:] == -1)
        np.testing.assert_array_equal(oracle.candidate_tokens(cand, cbs, ks, ke), sorted(toks))


# ------------------------------------------------------ candidate source ---------

@pytest.mark.parametrize("chunk", range(4))
def test_source_candidates_match_brute_force(chunk):
    """The source layer's publication against the brute force (dense logits with numpy,
    block maxima by reduceat, a full lexsort), exactly, in both scoring formats."""
    for i in range(chunk * 25, chunk * 25 + 25):
        rng = np.random.default_rng(7000 + i)
        spec = _tiny_spec(rng, i)
        case = W.generate(spec, seed=200 + i)
        pool = case.layers[0].host_pool(spec.page_bytes)
        nb = int(rng.integers(1, 12))
        sfmt = "bf16" if i % 3 == 0 else "fp32"
        width = 400
        for fmt in spec.q_formats:
            cand, score = oracle.source_candidates(case, nb=nb, q_format=fmt, pool=pool,
                                                   score_format=sfmt, score_width=width)
            for r in range(case.num_rows):
                want, wscores = brute_source_row(case, r, nb, q_format=fmt, pool=pool,
                                                 score_format=sfmt)
                np.testing.assert_array_equal(cand[r], want, err_msg=f"case {i} row {r}")
                got = {b: float(score[r, b]) for b in range(width) if not np.isnan(score[r, b])}
                assert got == wscores, f"case {i} row {r}"


def test_source_candidates_closed_form():
    # One head, weight 1; K zero except one token in each of blocks 2, 5, 6 with dots
    # 3 * 2^s (s = 1, 3, 2): block scores 6, 24, 12, every other block of the 8 scores 0.
    # nb = 2 -> blocks 5 and 6; nb = 4 -> 2, 5, 6 and the lowest zero block, 0.
    # With ks = 20 and ke = 90 the eligible blocks are 1..5 (block 1 = tokens 16..31 and
    # block 5 = tokens 80..95 only partly in range; block 0 lies below ks, block 6 at or
    # past ke); the block-5 token at t = 91 is past ke, so block 5 scores 0, and nb = 3
    # gives block 2 (6) and the two lowest of the zero-score blocks 1, 3, 4, 5: 1 and 3.
    case = _one_row_case(H=1, D=128, ps=16, n_tokens=128, cbs=16, nb=8, topk=4)
    L = case.layers[0]
    L.weights[:] = 1.0
    qv = np.zeros(64, np.uint8)
    qv[0] = 0x05                                         # element 0: 3.0
    L.q_values[0, 0] = qv
    for t, sc in ((33, 1), (91, 3), (100, 2)):           # blocks 2, 5, 6
        kv = np.zeros(64, np.uint8)
        kv[0] = 0x02                                     # element 0: 1.0
        _set_k(case, t, kv, np.array([127 + sc, 127, 127, 127], np.uint8))
    cand, score = oracle.source_candidates(case, nb=2, score_width=8)
    np.testing.assert_array_equal(cand[0], [5, 6])
    np.testing.assert_array_equal(score[0], [0, 0, 6, 0, 0, 24, 12, 0])
    cand, _ = oracle.source_candidates(case, nb=4)
    np.testing.assert_array_equal(cand[0], [0, 2, 5, 6])
    case.row_ks[0], case.row_ke[0] = 20, 90
    cand, score = oracle.source_candidates(case, nb=3, score_width=8)
    np.testing.assert_array_equal(cand[0], [1, 2, 3])
    assert np.isnan(score[0, 0]) and np.isnan(score[0, 6]) and np.isnan(score[0, 7])
    np.testing.assert_array_equal(score[0, 1:6], [0, 6, 0, 0, 0])


def test_source_candidates_invariants():
    for i in range(30):
        spec = W.Spec(name="si", num_rows=3, num_heads=2, head_dim=32, page_size=8, cbs=8, nb=6,
                      topk=4, ke_rule="uniform", ke_lo=0, ke_hi=120, ks_rule="random",
                      cand_rule="distinct", fill="all")
        case = W.generate(spec, i)
        nb = 1 + i % 9
        cand, score = oracle.source_candidates(case, nb=nb, score_width=16)
        for r in range(case.num_rows):
            ks, ke = int(case.row_ks[r]), int(case.row_ke[r])
            eligible = [b for b in range(16) if max(b * 8, ks) < min(b * 8 + 8, ke)]
            count = min(nb, len(eligible))
            assert np.all(cand[r, count:] == -1)
            chosen = cand[r, :count]
            assert np.all(np.diff(chosen) > 0) and set(chosen) <= set(eligible)
            rest = [b for b in eligible if b not in set(chosen)]
            if count and rest:
                lo = min(score[r, b] for b in chosen)
                hi = max(score[r, b] for b in rest)
                assert lo >= hi
                if lo == hi:
                    assert max(b for b in chosen if score[r, b] == lo) < \
                        min(b for b in rest if score[r, b] == hi)
