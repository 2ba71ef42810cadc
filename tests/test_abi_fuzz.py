"""Property tests of the host-side configuration rules and size queries (no launches): any
configuration is either rejected with a negative status and a message, or accepted with
every documented invariant holding, and the size queries agree with their formulas."""
import ctypes

from hypothesis import given, settings
from hypothesis import strategies as st

import sparse_attention_indexer_candidate_amd as idx

INT32 = st.integers(min_value=-2**31, max_value=2**31 - 1)


def near(*values):
    """Mostly the interesting values, sometimes any int32."""
    return st.one_of(st.sampled_from(values), INT32)


CONFIGS = st.builds(
    idx.idx_config,
    near(64, 32, 0, 128),                       # num_heads
    near(128, 64, 0, 256),                      # head_dim
    near(0, 1, 2, -1),                          # q_format
    near(16, 32, 64, 128, 256, 48, 0, 8192),    # page_size
    near(16, 32, 64, 128, 192, 256, 48, 8, 0),  # candidate_block_size
    near(0, 16, 32, 64, 128, 48),               # sparse_block_kv
    near(1, 8, 64, 128, 129, 512, 0, 4096),     # num_candidate_blocks
    near(1, 100, 2048, 4096, 8192, 8193, 0),    # topk
    near(0, 1, 2, -1),                          # score_format
)


@settings(max_examples=400, deadline=None)
@given(CONFIGS)
def test_config_rules(c):
    before = [getattr(c, f) for f, _ in idx.idx_config._fields_]
    rc = idx.lib.idx_check_config(ctypes.byref(c))
    if rc != idx.IDX_OK:
        assert rc in (idx.IDX_EINVAL, idx.IDX_EUNSUPPORTED)
        assert idx.idx_last_error()
        assert [getattr(c, f) for f, _ in idx.idx_config._fields_] == before   # untouched
        assert idx.lib.idx_num_sparse_blocks(ctypes.byref(c)) == rc
        assert idx.idx_schedule_work_bytes(c, 4) == 0 and idx.idx_workspace_bytes(c, 4, 0) == 0
        return
    assert idx.idx_last_error() == ""
    assert (c.num_heads, c.head_dim) == (64, 128)
    assert c.q_format in (0, 1) and c.score_format in (0, 1)
    sbk, cbs, nb = c.sparse_block_kv, c.candidate_block_size, c.num_candidate_blocks
    assert sbk in (16, 32, 64) and cbs % sbk == 0 and c.page_size % sbk == 0
    if before[5] == 0:                                   # chosen: 64 if possible, else cbs
        assert sbk == (64 if cbs % 64 == 0 else cbs)
    else:
        assert sbk == before[5]
    assert 1 <= nb * cbs <= idx.IDX_MAX_ROW_COLS
    assert 1 <= c.topk <= min(nb * cbs, idx.IDX_MAX_TOPK)
    nsb = idx.idx_num_sparse_blocks(c)
    assert nsb == nb * cbs // sbk
    assert idx.idx_workspace_bytes(c, 3, 0) == 3 * nb * cbs * 4
    assert idx.idx_workspace_bytes(c, 3, 100000) == 3 * ((100000 + 63) // 64 * 64) * 4
    assert idx.idx_schedule_work_bytes(c, 5) >= 5 * (1 + nsb) * 4   # kept + pages
    assert idx.idx_schedule_work_bytes(c, -1) == 0


@settings(max_examples=200, deadline=None)
@given(st.integers(min_value=-5, max_value=70000), st.integers(min_value=-5, max_value=2**20),
       st.sampled_from([16, 32, 64, 128, 256]))
def test_publish_workspace_sizes(max_rows, max_ctx, cbs):
    c = idx.make_config(page_size=256, candidate_block_size=cbs, num_candidate_blocks=1, topk=1)
    got = idx.idx_publish_workspace_bytes(c, max_rows, max_ctx)
    if max_rows < 0 or max_ctx <= 0:
        assert got == 0
        return
    part = min(cbs, 64)
    assert got >= max_rows * ((max_ctx + part - 1) // part) * 4
