"""The C-ABI library on the CPU: it loads, exports every declared symbol, applies the
configuration rules, and rejects bad arguments on the host before any launch.

No test here reaches a kernel launch: each call either fails a host check or has
zero rows (which launches nothing), so fake pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import sparse_attention_indexer_candidate_amd as idx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000          # 16-byte aligned, never dereferenced


def declared_functions():
    src = open(os.path.join(ROOT, "include", "idx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert names == sorted(idx.EXPORTED), names
    lib = ctypes.CDLL(idx.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_build_compiles_every_kernel_source():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_idx_build_check", os.path.join(ROOT, "sparse_attention_indexer_candidate_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    csrc = os.path.join(ROOT, "sparse_attention_indexer_candidate_amd", "csrc")
    on_disk = sorted("csrc/" + n for n in os.listdir(csrc) if n.endswith(".hip"))
    assert sorted(b.SOURCES) == on_disk


def test_header_is_c99_and_struct_layouts_match_the_binding(tmp_path):
    """include/idx.h compiles as plain C99 and each struct's size and field offsets in C
    equal the ctypes mirror's."""
    import subprocess

    structs = ["idx_config", "idx_kcache", "idx_rows", "idx_schedule", "idx_layer",
               "idx_plan_info"]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "idx.h"', "int main(void) {"]
    for name in structs:
        lines.append(f'    printf("{name} %zu\\n", sizeof({name}));')
        for f, _ in getattr(idx, name)._fields_:
            lines.append(f'    printf("{name}.{f} %zu\\n", offsetof({name}, {f}));')
    lines += ["    return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    for name in structs:
        st = getattr(idx, name)
        assert int(got[name]) == ctypes.sizeof(st), name
        for f, _ in st._fields_:
            assert int(got[f"{name}.{f}"]) == getattr(st, f).offset, f"{name}.{f}"


def test_readme_c_example_compiles_against_the_header(tmp_path):
    """The README's C call sequence stays valid C99 against include/idx.h."""
    import subprocess

    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```c\n(.*?)```", text, re.S).group(1)
    decls = ("int32_t max_rows = 64, n = 64; int64_t page_bytes = 4352, num_pages = 100;\n"
             "int64_t table_stride = 128; int32_t num_tables = 64, pages_per_table = 128;\n"
             "void *d_ks = 0, *d_ke = 0, *d_table = 0, *d_values = 0, *d_scales = 0,\n"
             "     *d_block_table = 0, *d_sparse_indices = 0, *d_end = 0, *d_work = 0,\n"
             "     *d_candidates = 0, *d_q_values = 0, *d_q_scales = 0, *d_weights = 0,\n"
             "     *d_topk = 0, *d_ws = 0, *stream = 0;\n")
    src = tmp_path / "readme.c"
    src.write_text('#include <stddef.h>\n#include <stdint.h>\n#include "idx.h"\nint main(void) {\n'
                   + decls + code + "(void)nsb;\nreturn 0;\n}\n")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-Wno-unused-variable",
                    "-fsyntax-only", "-I", os.path.join(ROOT, "include"), str(src)], check=True)


def cfg(**kw):
    base = dict(num_heads=64, head_dim=128, q_format=0, page_size=64, candidate_block_size=64,
                sparse_block_kv=0, num_candidate_blocks=64, topk=2048, score_format=0)
    base.update(kw)
    return idx.idx_config(*[base[f] for f, _ in idx.idx_config._fields_])


@pytest.mark.parametrize("cbs,want", [(64, 64), (128, 64), (192, 64), (16, 16), (32, 32)])
def test_sparse_block_pick(cbs, want):
    c = cfg(candidate_block_size=cbs, num_candidate_blocks=8, topk=8, page_size=128)
    idx.idx_check_config(c)
    assert c.sparse_block_kv == want
    assert idx.idx_num_sparse_blocks(c) == 8 * cbs // want


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads=32), idx.IDX_EUNSUPPORTED),
    (dict(head_dim=64), idx.IDX_EUNSUPPORTED),
    (dict(q_format=7), idx.IDX_EINVAL),
    (dict(score_format=2), idx.IDX_EINVAL),
    (dict(score_format=-1), idx.IDX_EINVAL),
    (dict(candidate_block_size=0), idx.IDX_EINVAL),
    (dict(num_candidate_blocks=0), idx.IDX_EINVAL),
    (dict(candidate_block_size=48), idx.IDX_EUNSUPPORTED),
    (dict(candidate_block_size=8), idx.IDX_EUNSUPPORTED),
    (dict(sparse_block_kv=48), idx.IDX_EUNSUPPORTED),
    (dict(sparse_block_kv=128, candidate_block_size=128), idx.IDX_EUNSUPPORTED),
    (dict(page_size=96), idx.IDX_EINVAL),          # not a multiple of sbk = 64
    (dict(page_size=0), idx.IDX_EINVAL),
    (dict(topk=0), idx.IDX_EINVAL),
    (dict(topk=4097), idx.IDX_EINVAL),             # > NB * cbs = 4096
    (dict(num_candidate_blocks=129), idx.IDX_EUNSUPPORTED),  # 129 * 64 > 8192 columns
])
def test_config_errors(kw, code):
    c = cfg(**kw)
    with pytest.raises(idx.IdxError) as e:
        idx.idx_check_config(c)
    assert e.value.code == code
    assert idx.idx_last_error()


def test_explicit_sparse_block_kept():
    c = cfg(candidate_block_size=64, sparse_block_kv=32, page_size=32)
    idx.idx_check_config(c)
    assert c.sparse_block_kv == 32 and idx.idx_num_sparse_blocks(c) == 128


def test_sizes():
    c = idx.idx_check_config(cfg())
    assert idx.idx_workspace_bytes(c, 64, 0) == 64 * 4096 * 4
    assert idx.idx_workspace_bytes(c, 128, 65536) == 128 * 65536 * 4
    assert idx.idx_workspace_bytes(c, 2, 100) == 2 * 4096 * 4      # sparse need dominates
    assert idx.idx_workspace_bytes(c, 2, 5000) == 2 * 5056 * 4     # dense rounds to 64
    assert idx.idx_schedule_work_bytes(c, 64) >= 64 * 4
    assert idx.idx_workspace_bytes(cfg(num_heads=1), 4, 0) == 0


def test_size_queries_return_zero_on_bad_input():
    c = idx.idx_check_config(cfg())
    assert idx.idx_schedule_work_bytes(c, -1) == 0
    assert idx.idx_schedule_work_bytes(cfg(num_heads=1), 4) == 0
    assert idx.idx_publish_workspace_bytes(cfg(num_heads=1), 4, 1024) == 0


def test_last_error_is_per_thread():
    """Each thread reads the message of its own last failing call; a thread with no
    failure reads "", and other threads' failures leave it unchanged."""
    import threading

    def fail_with(**kw):
        return idx.lib.idx_check_config(ctypes.byref(cfg(**kw)))

    assert fail_with(topk=0) != idx.IDX_OK
    main_msg = idx.idx_last_error()
    assert main_msg
    seen = {}

    def worker(name, kw):
        if kw is not None:
            assert fail_with(**kw) != idx.IDX_OK
        seen[name] = idx.idx_last_error()

    threads = [threading.Thread(target=worker, args=("heads", dict(num_heads=1))),
               threading.Thread(target=worker, args=("dim", dict(head_dim=64))),
               threading.Thread(target=worker, args=("none", None))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert seen["none"] == ""
    assert seen["heads"] and seen["dim"] and seen["heads"] != seen["dim"]
    assert main_msg not in (seen["heads"], seen["dim"])
    assert idx.idx_last_error() == main_msg


def test_timing_events_need_both_or_neither():
    assert idx.lib.idx_set_timing_events(FAKE, None) == idx.IDX_EINVAL
    assert idx.lib.idx_set_timing_events(None, FAKE) == idx.IDX_EINVAL
    assert idx.lib.idx_set_timing_events(None, None) == idx.IDX_OK


# ----------------------------------------------------------- call argument checks --

def kcache(**kw):
    base = dict(values=FAKE, values_page_stride=4352, scales=FAKE + 4096, scales_page_stride=4352,
                num_pages=10, block_table=FAKE, block_table_stride=4, num_tables=2,
                pages_per_table=4)
    base.update(kw)
    return idx.idx_kcache(*[base[f] for f, _ in idx.idx_kcache._fields_])


def rows(n=2, **kw):
    base = dict(num_rows=n, row_ks=None, row_ke=FAKE, row_table=None, rows_per_request=1)
    base.update(kw)
    return idx.idx_rows(*[base[f] for f, _ in idx.idx_rows._fields_])


def sched(work_bytes=1024, **kw):
    base = dict(sparse_indices=FAKE, end=FAKE, work=FAKE, work_bytes=work_bytes)
    base.update(kw)
    return idx.idx_schedule(*[base[f] for f, _ in idx.idx_schedule._fields_])


def sparse_call(c=None, r=None, k=None, s=None, qv=FAKE, qs=FAKE, w=FAKE, out=FAKE, ostride=2048,
                logits=None, ws=None, wsb=0):
    c = c or idx.idx_check_config(cfg())
    return idx.lib.idx_sparse_mqa_logits_topk(
        ctypes.byref(c), ctypes.byref(r or rows()), qv, qs, w, ctypes.byref(k or kcache()),
        ctypes.byref(s or sched()), out, ostride, logits, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(qv=None), idx.IDX_EINVAL),
    (dict(qv=FAKE + 4), idx.IDX_EINVAL),                 # q_values not 16-byte aligned
    (dict(w=None), idx.IDX_EINVAL),
    (dict(out=None), idx.IDX_EINVAL),
    (dict(ostride=100), idx.IDX_EINVAL),                 # out_stride < topk
    (dict(), idx.IDX_EWORKSPACE),                        # no logits buffer, no workspace
    (dict(ws=FAKE, wsb=1000), idx.IDX_EWORKSPACE),        # workspace too small
    (dict(s=sched(work_bytes=4)), idx.IDX_EWORKSPACE),   # schedule work too small for 2 rows
    (dict(s=sched(end=None)), idx.IDX_EINVAL),
    (dict(r=rows(-1)), idx.IDX_EINVAL),
    (dict(r=rows(2, row_ke=None)), idx.IDX_EINVAL),
    (dict(r=rows(2, rows_per_request=-1)), idx.IDX_EINVAL),
    (dict(k=kcache(values=None)), idx.IDX_EINVAL),
    (dict(k=kcache(num_pages=0)), idx.IDX_EINVAL),
    (dict(k=kcache(block_table_stride=2)), idx.IDX_EINVAL),
    (dict(k=kcache(values_page_stride=100)), idx.IDX_EINVAL),
    (dict(k=kcache(values=FAKE + 8)), idx.IDX_EINVAL),
])
def test_sparse_call_rejects_bad_arguments(kw, code):
    assert sparse_call(**kw) == code
    assert idx.idx_last_error()


def test_unchecked_config_is_rejected():
    c = cfg()   # sparse_block_kv still 0
    assert sparse_call(c=c, logits=FAKE) == idx.IDX_EINVAL
    assert "idx_check_config" in idx.idx_last_error()


def test_zero_rows_launch_nothing_and_succeed():
    assert sparse_call(r=rows(0), logits=FAKE) == idx.IDX_OK
    assert idx.idx_last_error() == ""
    c = idx.idx_check_config(cfg())
    rc = idx.lib.idx_expand_candidates(ctypes.byref(c), ctypes.byref(rows(0)),
                                       ctypes.byref(kcache()), FAKE, 64, ctypes.byref(sched()),
                                       None)
    assert rc == idx.IDX_OK


def test_expand_rejects_bad_arguments():
    c = idx.idx_check_config(cfg())
    call = lambda cand, stride, s=None: idx.lib.idx_expand_candidates(
        ctypes.byref(c), ctypes.byref(rows()), ctypes.byref(kcache()), cand, stride,
        ctypes.byref(s or sched()), None)
    assert call(None, 64) == idx.IDX_EINVAL
    assert call(FAKE, 10) == idx.IDX_EINVAL            # stride < NB
    assert call(FAKE, 64, sched(sparse_indices=None)) == idx.IDX_EINVAL


def layers_call(layers, n=None, r=None, ws=None, wsb=0, ostride=2048):
    c = idx.idx_check_config(cfg())
    arr = (idx.idx_layer * max(1, len(layers)))(*layers)
    return idx.lib.idx_sparse_mqa_logits_topk_layers(
        ctypes.byref(c), ctypes.byref(r or rows()), ctypes.byref(sched()),
        len(layers) if n is None else n, arr, ostride, ws, wsb, None)


def layer(k=None, qv=FAKE, out=FAKE, logits=FAKE):
    return idx.idx_layer(qv, FAKE, FAKE, k or kcache(), out, logits)


def test_layers_call_rejects_bad_arguments():
    two = [layer(), layer(kcache(values=FAKE + 0x10000, scales=FAKE + 0x11000))]
    assert layers_call(two, r=rows(0)) == idx.IDX_OK           # zero rows: nothing launched
    assert layers_call(two, n=0) == idx.IDX_EINVAL
    assert layers_call([layer()] * 9) == idx.IDX_EINVAL         # > IDX_MAX_LAYERS
    assert layers_call(two, ostride=100) == idx.IDX_EINVAL
    c = idx.idx_check_config(cfg())
    assert idx.lib.idx_sparse_mqa_logits_topk_layers(
        ctypes.byref(c), ctypes.byref(rows()), ctypes.byref(sched()), 2, None, 2048, None, 0,
        None) == idx.IDX_EINVAL
    # per-layer checks name the layer
    assert layers_call([layer(), layer(qv=FAKE + 4)]) == idx.IDX_EINVAL
    assert "layer 1" in idx.idx_last_error()
    assert layers_call([layer(), layer(out=None)]) == idx.IDX_EINVAL
    assert layers_call([layer(), layer(k=kcache(values=None))]) == idx.IDX_EINVAL
    assert "layer 1" in idx.idx_last_error()
    # one page geometry and block table for every layer
    for kw in (dict(num_pages=11), dict(block_table=FAKE + 0x100), dict(values_page_stride=4368),
               dict(pages_per_table=3)):
        assert layers_call([layer(), layer(k=kcache(**kw))]) == idx.IDX_EINVAL, kw
        assert "geometry" in idx.idx_last_error()
    # a layer without logits_out needs the workspace
    assert layers_call([layer(), layer(logits=None)]) == idx.IDX_EWORKSPACE
    assert layers_call([layer(), layer(logits=None)], ws=FAKE, wsb=100) == idx.IDX_EWORKSPACE


def expand_score_call(layers, cand=FAKE, stride=64, n=None, r=None, ws=None, wsb=0,
                      ostride=2048, s=None):
    c = idx.idx_check_config(cfg())
    arr = (idx.idx_layer * max(1, len(layers)))(*layers)
    return idx.lib.idx_expand_and_score_layers(
        ctypes.byref(c), ctypes.byref(r or rows()), cand, stride, ctypes.byref(s or sched()),
        len(layers) if n is None else n, arr, ostride, ws, wsb, None)


def test_expand_and_score_rejects_what_either_call_rejects():
    """idx_expand_and_score_layers applies the checks of idx_expand_candidates (candidate
    ids, their stride, the schedule) and of idx_sparse_mqa_logits_topk_layers (layers,
    outputs, one cache geometry, the workspace), on the host before any launch."""
    two = [layer(), layer(kcache(values=FAKE + 0x10000, scales=FAKE + 0x11000))]
    assert expand_score_call(two, r=rows(0)) == idx.IDX_OK        # zero rows: nothing launched
    assert expand_score_call(two, r=rows(0), cand=None) == idx.IDX_OK
    assert expand_score_call(two, cand=None) == idx.IDX_EINVAL
    assert "candidate_blocks" in idx.idx_last_error()
    assert expand_score_call(two, stride=10) == idx.IDX_EINVAL    # stride < NB
    assert "cand_stride" in idx.idx_last_error()
    assert expand_score_call(two, s=sched(sparse_indices=None)) == idx.IDX_EINVAL
    assert expand_score_call(two, n=0) == idx.IDX_EINVAL
    assert expand_score_call([layer()] * 9) == idx.IDX_EINVAL    # > IDX_MAX_LAYERS
    assert expand_score_call(two, ostride=100) == idx.IDX_EINVAL
    assert expand_score_call([layer(), layer(qv=FAKE + 4)]) == idx.IDX_EINVAL
    assert "layer 1" in idx.idx_last_error()
    assert expand_score_call([layer(), layer(k=kcache(num_pages=11))]) == idx.IDX_EINVAL
    assert "geometry" in idx.idx_last_error()
    assert expand_score_call([layer(), layer(logits=None)]) == idx.IDX_EWORKSPACE
    c = idx.idx_check_config(cfg())
    assert idx.lib.idx_expand_and_score_layers(
        ctypes.byref(c), ctypes.byref(rows()), FAKE, 64, ctypes.byref(sched()), 2, None, 2048,
        None, 0, None) == idx.IDX_EINVAL


def test_gather_rejects_bad_arguments():
    c = idx.idx_check_config(cfg())
    def call(k=None, n=2, cu=FAKE, seq=100, tokens=500, vo=FAKE, so=FAKE):
        return idx.lib.idx_gather_k_workspace(ctypes.byref(c), ctypes.byref(k or kcache()), n, cu,
                                              None, seq, tokens, vo, so, None)
    assert call(n=0) == idx.IDX_OK                   # nothing to gather: no launch
    assert call(seq=0) == idx.IDX_OK
    assert call(n=-1) == idx.IDX_EINVAL
    assert call(n=70000) == idx.IDX_EUNSUPPORTED     # one grid row per request
    assert call(cu=None) == idx.IDX_EINVAL
    assert call(vo=None) == idx.IDX_EINVAL
    assert call(vo=FAKE + 4) == idx.IDX_EINVAL       # values_out not 16-byte aligned
    assert call(so=FAKE + 2) == idx.IDX_EINVAL       # scales_out not 4-byte aligned
    assert call(k=kcache(scales=FAKE + 4098)) == idx.IDX_EINVAL
    assert call(k=kcache(values=None)) == idx.IDX_EINVAL
    assert idx.lib.idx_gather_k_workspace(ctypes.byref(cfg()), ctypes.byref(kcache()), 1, FAKE,
                                          None, 1, 1, FAKE, FAKE, None) == idx.IDX_EINVAL


def test_gather_binding_checks_workspace_shapes():
    import torch

    c = idx.idx_check_config(cfg())
    cu = torch.zeros(2, dtype=torch.int32)
    for vals, scs in ((torch.empty(10, 64, dtype=torch.uint8), torch.empty(9, 4, dtype=torch.uint8)),
                      (torch.empty(10, 32, dtype=torch.uint8), torch.empty(10, 4, dtype=torch.uint8)),
                      (torch.empty(64, 10, dtype=torch.uint8).t(), torch.empty(10, 4, dtype=torch.uint8))):
        with pytest.raises(ValueError):
            idx.idx_gather_k_workspace(c, kcache(), cu, vals, scs, 1)


def test_dense_call_rejects_bad_arguments():
    c = idx.idx_check_config(cfg())
    def call(max_ctx=65536, logits=None, lstride=0, ws=None, wsb=0):
        return idx.lib.idx_dense_masked_logits_topk(
            ctypes.byref(c), ctypes.byref(rows()), max_ctx, FAKE, FAKE, FAKE,
            ctypes.byref(kcache()), ctypes.byref(sched()), FAKE, 2048, logits, lstride, ws, wsb,
            None)
    assert call(max_ctx=0) == idx.IDX_EUNSUPPORTED
    assert call(max_ctx=65537) == idx.IDX_EUNSUPPORTED
    assert call() == idx.IDX_EWORKSPACE
    assert call(logits=FAKE, lstride=1000) == idx.IDX_EINVAL
    assert call(ws=FAKE, wsb=16) == idx.IDX_EWORKSPACE


def test_one_hip_runtime_per_process():
    """Importing the binding before torch must not map a second HIP runtime (ROCm's
    libamdhip64 beside torch's): kernels launched through the second one see no device."""
    import subprocess
    import sys
    code = ("import sparse_attention_indexer_candidate_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout


def test_bound_calls_check_arguments_like_the_wrappers():
    """Calls bound ahead of time pass the same arguments to the same C entry points."""
    c = idx.idx_check_config(cfg())
    ok = idx.bind_sparse_mqa_logits_topk(c, rows(0), FAKE, FAKE, FAKE, kcache(), sched(), FAKE,
                                         2048, FAKE)
    assert ok() == idx.IDX_OK   # zero rows: nothing to launch
    bad = idx.bind_sparse_mqa_logits_topk(c, rows(2), None, FAKE, FAKE, kcache(), sched(), FAKE,
                                          2048, FAKE)
    with pytest.raises(idx.IdxError) as e:
        bad()
    assert e.value.code == idx.IDX_EINVAL
    short = idx.bind_sparse_mqa_logits_topk(c, rows(2), FAKE, FAKE, FAKE, kcache(), sched(), FAKE,
                                            2048, None, FAKE, 1000)
    with pytest.raises(idx.IdxError) as e:
        short()
    assert e.value.code == idx.IDX_EWORKSPACE
    assert idx.bind_expand_candidates(c, rows(0), kcache(), FAKE, 64, sched())() == idx.IDX_OK
    dense = idx.bind_dense_masked_logits_topk(c, rows(2), 0, FAKE, FAKE, FAKE, kcache(), sched(),
                                              FAKE, 2048, FAKE, 0)
    with pytest.raises(idx.IdxError):
        dense()


def test_fp8_dot_measurement_rejects_bad_arguments():
    for args in [(None, FAKE, FAKE, 0, FAKE), (FAKE, FAKE, FAKE, 3, FAKE), (FAKE, FAKE, FAKE, -1, FAKE),
                 (FAKE + 4, FAKE, FAKE, 0, FAKE), (FAKE, FAKE, FAKE, 1, None)]:
        with pytest.raises(idx.IdxError) as e:
            idx.idx_measure_fp8_dot(*args)
        assert e.value.code == idx.IDX_EINVAL


def test_measurement_kernels_reject_bad_arguments_on_the_host():
    with pytest.raises(idx.IdxError) as e:
        idx.idx_measure_read(FAKE, 17, FAKE)          # not a multiple of 16 bytes
    assert e.value.code == idx.IDX_EINVAL
    with pytest.raises(idx.IdxError):
        idx.idx_measure_read(FAKE + 4, 64, FAKE)      # src not 16-byte aligned
    with pytest.raises(idx.IdxError):
        idx.idx_measure_read(None, 64, FAKE)
    with pytest.raises(idx.IdxError) as e:
        idx.idx_measure_mfma(0, FAKE)
    assert e.value.code == idx.IDX_EINVAL
    with pytest.raises(idx.IdxError):
        idx.idx_measure_mfma(16, None)
    with pytest.raises(idx.IdxError) as e:
        idx.idx_measure_mfma_relu(0, FAKE)
    assert e.value.code == idx.IDX_EINVAL
    with pytest.raises(idx.IdxError):
        idx.idx_measure_mfma_relu(16, FAKE + 2)
    # waves x rounds x 8 chains x 16*16*128 multiply-adds x 2
    assert idx.idx_measure_mfma_flops(3) == idx.IDX_MEASURE_WGS * 4 * 3 * 8 * 16 * 16 * 128 * 2


def test_sparse_plan_rule_on_the_host():
    """The launch plan for each row / layer count (host only: without a GPU the CU count
    query falls back to 256, the MI355X's).  The rule: MXFP4 queries, 64-token sparse
    blocks and >= 8 rows per CU take row groups; >= 1 row per CU one workgroup a row;
    fewer rows but at least one row-layer per CU one workgroup a row-layer; fewer still
    split rows over workgroups, all layers in one launch pair only when every layer's
    logits have a home."""
    c = idx.make_config()
    cus = 256
    want = [
        (0, 1, False, idx.IDX_PLAN_NONE, ""),
        (64, 1, False, idx.IDX_PLAN_SPLIT, "score_split_kernel"),
        (cus - 1, 4, True, idx.IDX_PLAN_ONE_ROW_LAYERS, "fused_layers_kernel"),
        (64, 4, False, idx.IDX_PLAN_ONE_ROW_LAYERS, "fused_layers_kernel"),
        (32, 8, True, idx.IDX_PLAN_ONE_ROW_LAYERS, "fused_layers_kernel"),
        (63, 4, True, idx.IDX_PLAN_SPLIT_LAYERS, "score_split_layers_kernel"),
        (63, 4, False, idx.IDX_PLAN_SPLIT, "score_split_kernel"),
        (cus, 1, False, idx.IDX_PLAN_ONE_ROW, "fused_row_kernel"),
        (cus, 4, False, idx.IDX_PLAN_ONE_ROW_LAYERS, "fused_layers_kernel"),
        (8 * cus - 1, 1, False, idx.IDX_PLAN_ONE_ROW, "fused_row_kernel"),
        (8 * cus, 1, False, idx.IDX_PLAN_ROW_GROUP, "row_group_kernel"),
        (4096, 2, False, idx.IDX_PLAN_ROW_GROUP_LAYERS, "row_group_layers_kernel"),
    ]
    for rows, layers, home, plan, kernel in want:
        p = idx.idx_sparse_plan(c, rows, layers, home)
        assert (p["plan"], p["scoring_kernel"]) == (plan, kernel), (rows, layers, home, p)
        fused = plan in (idx.IDX_PLAN_ONE_ROW, idx.IDX_PLAN_ROW_GROUP, idx.IDX_PLAN_ONE_ROW_LAYERS,
                         idx.IDX_PLAN_ROW_GROUP_LAYERS)
        assert p["selects_in_scoring_kernel"] == fused
        assert p["selection_kernel"] == ("" if fused or plan == idx.IDX_PLAN_NONE else
                                         p["scoring_kernel"].replace("score_", "topk_"))
        multi = plan in (idx.IDX_PLAN_SPLIT_LAYERS, idx.IDX_PLAN_ONE_ROW_LAYERS,
                         idx.IDX_PLAN_ROW_GROUP_LAYERS)
        assert p["layers_per_scoring_launch"] == (0 if plan == idx.IDX_PLAN_NONE else
                                                  layers if multi else 1)
        # idx_expand_and_score_layers expands inside the one-row kernels (MXFP4, sbk 64,
        # NB <= 128) when they take every row-layer in one round (at most two a CU), and
        # inside the split scoring launch (one layer, or all layers in one launch pair);
        # else it keeps the expansion launch and the same scoring kernel
        if plan in (idx.IDX_PLAN_ONE_ROW, idx.IDX_PLAN_ONE_ROW_LAYERS) and rows * layers <= 2 * cus:
            want_kernel = "expand_" + kernel
        elif ((plan == idx.IDX_PLAN_SPLIT and layers == 1) or plan == idx.IDX_PLAN_SPLIT_LAYERS) \
                and rows * layers * 8 <= 6 * cus:   # 4096 columns: 8 workgroups a row
            want_kernel = kernel.replace("score_split_", "score_split_expand_")
        else:
            want_kernel = kernel
        assert p["expand_and_score_kernel"] == want_kernel, p
        assert p["expansion_in_scoring_kernel"] == (want_kernel != kernel), p
    # fp8 queries and 32-token sparse blocks never take row groups
    c8 = idx.make_config(q_format=idx.IDX_Q_FP8_E4M3_ROWSCALE)
    assert idx.idx_sparse_plan(c8, 4096)["plan"] == idx.IDX_PLAN_ONE_ROW
    c32 = idx.make_config(candidate_block_size=32, num_candidate_blocks=64)
    assert idx.idx_sparse_plan(c32, 4096)["plan"] == idx.IDX_PLAN_ONE_ROW
    # ... nor expand inside the scoring kernel (64-token sparse blocks with at most 8192
    # columns a row mean at most 128 candidate blocks: two ids a lane)
    p = idx.idx_sparse_plan(c32, 200, 2)
    assert p["plan"] == idx.IDX_PLAN_ONE_ROW_LAYERS and not p["expansion_in_scoring_kernel"]
    assert p["expand_and_score_kernel"] == p["scoring_kernel"]
    # fp8 queries: inside the 8-wave one-row shapes (fewer than two row-layers a CU)
    assert idx.idx_sparse_plan(c8, 200, 2)["expand_and_score_kernel"] == "expand_fused_layers_kernel"
    assert idx.idx_sparse_plan(c8, 300, 1)["expand_and_score_kernel"] == "expand_fused_row_kernel"
    assert not idx.idx_sparse_plan(c8, 2 * cus, 1)["expansion_in_scoring_kernel"]
    assert not idx.idx_sparse_plan(c8, cus, 2)["expansion_in_scoring_kernel"]
    assert idx.idx_sparse_plan(c, 200, 2)["expansion_in_scoring_kernel"]
    # fp8 queries: inside the split launches with 64-token sparse blocks only
    assert idx.idx_sparse_plan(c8, 64, 1)["expand_and_score_kernel"] == "score_split_expand_kernel"
    c8_32 = idx.make_config(q_format=idx.IDX_Q_FP8_E4M3_ROWSCALE, candidate_block_size=32)
    assert not idx.idx_sparse_plan(c8_32, 64, 1)["expansion_in_scoring_kernel"]
    # ... and only when every split workgroup is resident at once (three a CU for fp8, six
    # for MXFP4; 4096 columns are 8 workgroups a row)
    assert idx.idx_sparse_plan(c8, 96, 1)["expansion_in_scoring_kernel"]
    assert not idx.idx_sparse_plan(c8, 97, 1)["expansion_in_scoring_kernel"]
    assert idx.idx_sparse_plan(c, 192, 1)["expansion_in_scoring_kernel"]
    assert not idx.idx_sparse_plan(c, 193, 1)["expansion_in_scoring_kernel"]
    assert idx.idx_sparse_plan(c, 2 * cus, 1)["expand_and_score_kernel"] == "expand_fused_row_kernel"
    assert not idx.idx_sparse_plan(c, 2 * cus + 1, 1)["expansion_in_scoring_kernel"]
    assert not idx.idx_sparse_plan(c, cus, 3)["expansion_in_scoring_kernel"]
    for bad in [(c, -1, 1), (c, 4, 0), (c, 4, idx.IDX_MAX_LAYERS + 1)]:
        with pytest.raises(idx.IdxError):
            idx.idx_sparse_plan(*bad)


def test_noalloc_call_checks_arguments_and_zero_rows_launch_nothing():
    """idx_sparse_mqa_logits_topk_noalloc applies the same host checks as the workspace
    form (no workspace argument), and zero rows succeed without touching a device."""
    c = idx.make_config()
    rows0 = idx.idx_rows(0, None, FAKE, None)
    k = idx.idx_kcache(FAKE, 64 * 64, FAKE, 64 * 4, 10, FAKE, 4, 1, 4)
    nsb = idx.idx_num_sparse_blocks(c)
    sched = idx.idx_schedule(FAKE, FAKE, FAKE, idx.idx_schedule_work_bytes(c, 4))
    call = lambda **kw: idx.idx_sparse_mqa_logits_topk_noalloc(
        c, kw.get("rows", rows0), FAKE, FAKE, FAKE, k, kw.get("sched", sched),
        kw.get("out", FAKE), kw.get("stride", 2048), kw.get("lout"))
    assert call() == idx.IDX_OK
    for kw, code in [(dict(out=None), idx.IDX_EINVAL), (dict(stride=100), idx.IDX_EINVAL),
                     (dict(lout=FAKE + 4), idx.IDX_EINVAL),
                     (dict(rows=idx.idx_rows(4, None, None, None)), idx.IDX_EINVAL),
                     (dict(rows=idx.idx_rows(4, None, FAKE, None),
                           sched=idx.idx_schedule(FAKE, FAKE, FAKE, 4)), idx.IDX_EWORKSPACE)]:
        with pytest.raises(idx.IdxError) as e:
            call(**kw)
        assert e.value.code == code, kw
    assert nsb == 64
    assert idx.IDX_NOALLOC_SCRATCH_BYTES >= 255 * 8192 * 4   # the split plan always fits


def test_bf16_weights_alignment_is_checked():
    """bf16 weights must be 8-byte aligned (fp32: 4); checked before any launch."""
    c = cfg(score_format=idx.IDX_SCORE_BF16)
    idx.idx_check_config(c)
    k = idx.idx_kcache(FAKE, 64 * 64, FAKE, 64 * 4, 10, FAKE, 4, 1, 4)
    sched = idx.idx_schedule(FAKE, FAKE, FAKE, idx.idx_schedule_work_bytes(c, 4))
    rows = idx.idx_rows(0, None, FAKE, None)
    for w, ok in [(FAKE, True), (FAKE + 8, True), (FAKE + 4, False), (FAKE + 2, False)]:
        call = lambda: idx.idx_sparse_mqa_logits_topk(c, rows, FAKE, FAKE, w, k, sched, FAKE,
                                                      2048, FAKE)
        if ok:
            assert call() == idx.IDX_OK
        else:
            with pytest.raises(idx.IdxError) as e:
                call()
            assert e.value.code == idx.IDX_EINVAL and "8-byte" in str(e.value)


def test_publish_call_checks_arguments_and_sizes():
    """idx_publish_candidates: every bad argument is rejected on the host; zero rows launch
    nothing; the workspace holds one uint32 per part of min(cbs, 64) tokens a row."""
    c = cfg(num_candidate_blocks=64, topk=64)
    idx.idx_check_config(c)
    assert idx.idx_publish_workspace_bytes(c, 128, 65536) == 128 * 1024 * 4
    c16 = cfg(candidate_block_size=16, num_candidate_blocks=64, topk=64)
    idx.idx_check_config(c16)
    assert idx.idx_publish_workspace_bytes(c16, 2, 100) == 2 * 2 * 4 * 4
    k = idx.idx_kcache(FAKE, 64 * 64, FAKE, 64 * 4, 10, FAKE, 4, 1, 4)
    rows0 = idx.idx_rows(0, None, FAKE, None)
    rows4 = idx.idx_rows(4, None, FAKE, None)

    def call(rows=rows0, max_ctx=4096, cand=FAKE, stride=64, lout=None, lstride=0,
             ws=FAKE, wsb=1 << 20, w=FAKE):
        return idx.idx_publish_candidates(c, rows, max_ctx, FAKE, FAKE, w, k, cand, stride,
                                          lout, lstride, ws, wsb)
    assert call() == idx.IDX_OK
    for kw, code in [(dict(max_ctx=0), idx.IDX_EUNSUPPORTED),
                     (dict(max_ctx=4096 * 64 + 1), idx.IDX_EUNSUPPORTED),
                     (dict(cand=None), idx.IDX_EINVAL), (dict(stride=63), idx.IDX_EINVAL),
                     (dict(lout=FAKE, lstride=100), idx.IDX_EINVAL),
                     (dict(rows=rows4, ws=None), idx.IDX_EWORKSPACE),
                     (dict(rows=rows4, wsb=4 * 64 * 4 - 4), idx.IDX_EWORKSPACE),
                     (dict(w=None), idx.IDX_EINVAL)]:
        with pytest.raises(idx.IdxError) as e:
            call(**kw)
        assert e.value.code == code, kw
