"""Python binding of libidx, the candidate-consuming sparse MQA-logits indexer for MI355X.

Argument marshalling only: every step of the indexer runs in the HIP kernels of
``libidx.so`` (built from ``csrc/`` by ``build.py``).  The functions carry the C
names of ``include/idx.h`` and take either ctypes structs / raw device pointers, or
torch tensors through the small helpers below (PyTorch supplies device memory and
the stream, nothing else).  Importing this package fails loudly when the library
has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libidx.so")

IDX_OK = 0
IDX_EINVAL = -1
IDX_EUNSUPPORTED = -2
IDX_EWORKSPACE = -3
IDX_EHIP = -4
IDX_Q_MXFP4 = 0
IDX_Q_FP8_E4M3_ROWSCALE = 1
IDX_SCORE_FP32 = 0
IDX_SCORE_BF16 = 1
IDX_MAX_ROW_COLS = 8192
IDX_MAX_DENSE_COLS = 65536
IDX_MAX_TOPK = 8192

EXPORTED = ("idx_check_config", "idx_num_sparse_blocks", "idx_schedule_work_bytes",
            "idx_workspace_bytes", "idx_last_error", "idx_set_timing_events",
            "idx_expand_candidates", "idx_sparse_mqa_logits_topk",
            "idx_sparse_mqa_logits_topk_layers", "idx_expand_and_score_layers",
            "idx_dense_masked_logits_topk",
            "idx_gather_k_workspace", "idx_sparse_plan", "idx_sparse_mqa_logits_topk_noalloc",
            "idx_publish_workspace_bytes", "idx_publish_candidates",
            "idx_measure_read", "idx_measure_mfma", "idx_measure_mfma_relu",
            "idx_measure_mfma_flops", "idx_measure_fp8_dot")
IDX_MEASURE_WGS = 4096
IDX_MAX_LAYERS = 8
IDX_NOALLOC_SCRATCH_BYTES = 8 << 20


class IdxError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


class idx_config(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_format", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("candidate_block_size", ctypes.c_int32), ("sparse_block_kv", ctypes.c_int32),
                ("num_candidate_blocks", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("score_format", ctypes.c_int32)]


class idx_kcache(ctypes.Structure):
    _fields_ = [("values", ctypes.c_void_p), ("values_page_stride", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("scales_page_stride", ctypes.c_int64),
                ("num_pages", ctypes.c_int64), ("block_table", ctypes.c_void_p),
                ("block_table_stride", ctypes.c_int64), ("num_tables", ctypes.c_int32),
                ("pages_per_table", ctypes.c_int32)]


class idx_rows(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int32), ("row_ks", ctypes.c_void_p),
                ("row_ke", ctypes.c_void_p), ("row_table", ctypes.c_void_p),
                ("rows_per_request", ctypes.c_int32)]


class idx_schedule(ctypes.Structure):
    _fields_ = [("sparse_indices", ctypes.c_void_p), ("end", ctypes.c_void_p),
                ("work", ctypes.c_void_p), ("work_bytes", ctypes.c_size_t)]


class idx_layer(ctypes.Structure):
    _fields_ = [("q_values", ctypes.c_void_p), ("q_scales", ctypes.c_void_p),
                ("weights", ctypes.c_void_p), ("k", idx_kcache),
                ("topk_indices", ctypes.c_void_p), ("logits_out", ctypes.c_void_p)]


IDX_PLAN_NONE = 0
IDX_PLAN_SPLIT = 1
IDX_PLAN_ONE_ROW = 2
IDX_PLAN_ROW_GROUP = 3
IDX_PLAN_SPLIT_LAYERS = 4
IDX_PLAN_ONE_ROW_LAYERS = 5
IDX_PLAN_ROW_GROUP_LAYERS = 6


class idx_plan_info(ctypes.Structure):
    _fields_ = [("plan", ctypes.c_int32), ("layers_per_scoring_launch", ctypes.c_int32),
                ("selects_in_scoring_kernel", ctypes.c_int32),
                ("scoring_kernel", ctypes.c_char_p), ("selection_kernel", ctypes.c_char_p),
                ("expansion_in_scoring_kernel", ctypes.c_int32),
                ("expand_and_score_kernel", ctypes.c_char_p)]


def _load():
    # One HIP runtime per process.  torch ships its own libamdhip64 under the same
    # soname as ROCm's; once torch is loaded, libidx.so binds to that copy.  Loading
    # libidx.so first would map ROCm's copy too, and the two runtimes do not share
    # streams or device state (the second one finds no device).
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python sparse_attention_indexer_candidate_amd/build.py` "
                          "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.idx_check_config.argtypes = [P(idx_config)]
    L.idx_check_config.restype = ctypes.c_int
    L.idx_num_sparse_blocks.argtypes = [P(idx_config)]
    L.idx_num_sparse_blocks.restype = i32
    L.idx_schedule_work_bytes.argtypes = [P(idx_config), i32]
    L.idx_schedule_work_bytes.restype = sz
    L.idx_workspace_bytes.argtypes = [P(idx_config), i32, i32]
    L.idx_workspace_bytes.restype = sz
    L.idx_last_error.argtypes = []
    L.idx_last_error.restype = ctypes.c_char_p
    L.idx_set_timing_events.argtypes = [vp, vp]
    L.idx_set_timing_events.restype = ctypes.c_int
    L.idx_expand_candidates.argtypes = [P(idx_config), P(idx_rows), P(idx_kcache), vp, i64,
                                        P(idx_schedule), vp]
    L.idx_expand_candidates.restype = ctypes.c_int
    L.idx_sparse_mqa_logits_topk.argtypes = [P(idx_config), P(idx_rows), vp, vp, vp,
                                             P(idx_kcache), P(idx_schedule), vp, i64, vp, vp, sz,
                                             vp]
    L.idx_sparse_mqa_logits_topk.restype = ctypes.c_int
    L.idx_sparse_mqa_logits_topk_noalloc.argtypes = [P(idx_config), P(idx_rows), vp, vp, vp,
                                                     P(idx_kcache), P(idx_schedule), vp, i64, vp,
                                                     vp]
    L.idx_sparse_mqa_logits_topk_noalloc.restype = ctypes.c_int
    L.idx_sparse_mqa_logits_topk_layers.argtypes = [P(idx_config), P(idx_rows), P(idx_schedule),
                                                    i32, P(idx_layer), i64, vp, sz, vp]
    L.idx_sparse_mqa_logits_topk_layers.restype = ctypes.c_int
    L.idx_expand_and_score_layers.argtypes = [P(idx_config), P(idx_rows), vp, i64,
                                              P(idx_schedule), i32, P(idx_layer), i64, vp, sz, vp]
    L.idx_expand_and_score_layers.restype = ctypes.c_int
    L.idx_dense_masked_logits_topk.argtypes = [P(idx_config), P(idx_rows), i32, vp, vp, vp,
                                               P(idx_kcache), P(idx_schedule), vp, i64, vp, i64,
                                               vp, sz, vp]
    L.idx_dense_masked_logits_topk.restype = ctypes.c_int
    L.idx_gather_k_workspace.argtypes = [P(idx_config), P(idx_kcache), i32, vp, vp, i32, i32,
                                         vp, vp, vp]
    L.idx_gather_k_workspace.restype = ctypes.c_int
    L.idx_publish_workspace_bytes.argtypes = [P(idx_config), i32, i32]
    L.idx_publish_workspace_bytes.restype = sz
    L.idx_publish_candidates.argtypes = [P(idx_config), P(idx_rows), i32, vp, vp, vp,
                                         P(idx_kcache), vp, i64, vp, i64, vp, sz, vp]
    L.idx_publish_candidates.restype = ctypes.c_int
    L.idx_sparse_plan.argtypes = [P(idx_config), i32, i32, i32, P(idx_plan_info)]
    L.idx_sparse_plan.restype = ctypes.c_int
    L.idx_measure_read.argtypes = [vp, sz, vp, vp]
    L.idx_measure_read.restype = ctypes.c_int
    L.idx_measure_mfma.argtypes = [i32, vp, vp]
    L.idx_measure_mfma.restype = ctypes.c_int
    L.idx_measure_mfma_relu.argtypes = [i32, vp, vp]
    L.idx_measure_mfma_relu.restype = ctypes.c_int
    L.idx_measure_fp8_dot.argtypes = [vp, vp, vp, i32, vp, vp]
    L.idx_measure_fp8_dot.restype = ctypes.c_int
    L.idx_measure_mfma_flops.argtypes = [i32]
    L.idx_measure_mfma_flops.restype = i64
    return L


lib = _load()


def idx_last_error() -> str:
    return lib.idx_last_error().decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise IdxError(rc, idx_last_error())
    return rc


# ------------------------------------------------------------- raw C calls --

def idx_set_timing_events(start_event=None, stop_event=None) -> int:
    """Record the given HIP events (torch.cuda.Event or raw handles) around the scoring
    launch of subsequent calls on this thread; no arguments clears the hook."""
    def handle(e):
        if e is None:
            return None
        if hasattr(e, "cuda_event"):
            if not e.cuda_event:   # torch creates the HIP event lazily on first record
                e.record()
            return e.cuda_event
        return int(e)
    return _check(lib.idx_set_timing_events(handle(start_event), handle(stop_event)))


def idx_check_config(cfg: idx_config) -> idx_config:
    _check(lib.idx_check_config(ctypes.byref(cfg)))
    return cfg


def idx_num_sparse_blocks(cfg: idx_config) -> int:
    return _check(lib.idx_num_sparse_blocks(ctypes.byref(cfg)))


def idx_schedule_work_bytes(cfg: idx_config, max_rows: int) -> int:
    return lib.idx_schedule_work_bytes(ctypes.byref(cfg), max_rows)


def idx_workspace_bytes(cfg: idx_config, max_rows: int, max_ctx: int = 0) -> int:
    return lib.idx_workspace_bytes(ctypes.byref(cfg), max_rows, max_ctx)


def idx_sparse_plan(cfg: idx_config, num_rows: int, num_layers: int = 1,
                    logits_home: bool = False) -> dict:
    """The launch plan the library takes for a sparse call of these sizes on the current
    device: plan id, scoring / selection kernel names, layers per scoring launch."""
    info = idx_plan_info()
    _check(lib.idx_sparse_plan(ctypes.byref(cfg), num_rows, num_layers, int(bool(logits_home)),
                               ctypes.byref(info)))
    return dict(plan=info.plan, layers_per_scoring_launch=info.layers_per_scoring_launch,
                selects_in_scoring_kernel=bool(info.selects_in_scoring_kernel),
                scoring_kernel=info.scoring_kernel.decode(),
                selection_kernel=info.selection_kernel.decode(),
                expansion_in_scoring_kernel=bool(info.expansion_in_scoring_kernel),
                expand_and_score_kernel=info.expand_and_score_kernel.decode())


def idx_expand_candidates(cfg, rows, k, candidate_blocks, cand_stride, sched, stream=None):
    return _check(lib.idx_expand_candidates(ctypes.byref(cfg), ctypes.byref(rows),
                                            ctypes.byref(k), _p(candidate_blocks), cand_stride,
                                            ctypes.byref(sched), _p(stream)))


def idx_sparse_mqa_logits_topk(cfg, rows, q_values, q_scales, weights, k, sched, topk_indices,
                               out_stride, logits_out=None, workspace=None, workspace_bytes=0,
                               stream=None):
    return _check(lib.idx_sparse_mqa_logits_topk(
        ctypes.byref(cfg), ctypes.byref(rows), _p(q_values), _p(q_scales), _p(weights),
        ctypes.byref(k), ctypes.byref(sched), _p(topk_indices), out_stride, _p(logits_out),
        _p(workspace), workspace_bytes, _p(stream)))


def idx_sparse_mqa_logits_topk_noalloc(cfg, rows, q_values, q_scales, weights, k, sched,
                                       topk_indices, out_stride, logits_out=None, stream=None):
    """idx_sparse_mqa_logits_topk without a workspace: the library's static per-GPU scratch
    holds the logits when the call needs them kept (allocates nothing)."""
    return _check(lib.idx_sparse_mqa_logits_topk_noalloc(
        ctypes.byref(cfg), ctypes.byref(rows), _p(q_values), _p(q_scales), _p(weights),
        ctypes.byref(k), ctypes.byref(sched), _p(topk_indices), out_stride, _p(logits_out),
        _p(stream)))


def make_layers(layers):
    """Host array of idx_layer from (q_values, q_scales, weights, kcache, topk_indices,
    logits_out or None) tuples."""
    arr = (idx_layer * len(layers))()
    for i, (qv, qs, w, k, out, lout) in enumerate(layers):
        arr[i] = idx_layer(_p(qv), _p(qs), _p(w), k, _p(out), _p(lout))
    return arr


def idx_sparse_mqa_logits_topk_layers(cfg, rows, sched, layers, out_stride, workspace=None,
                                      workspace_bytes=0, stream=None):
    """layers: a make_layers() array (or tuples for it); every layer in one call."""
    arr = layers if isinstance(layers, ctypes.Array) else make_layers(layers)
    return _check(lib.idx_sparse_mqa_logits_topk_layers(
        ctypes.byref(cfg), ctypes.byref(rows), ctypes.byref(sched), len(arr), arr, out_stride,
        _p(workspace), workspace_bytes, _p(stream)))


def idx_expand_and_score_layers(cfg, rows, candidate_blocks, cand_stride, sched, layers,
                                out_stride, workspace=None, workspace_bytes=0, stream=None):
    """idx_expand_candidates (with layers[0]'s cache) then idx_sparse_mqa_logits_topk_layers
    in one call; layers as for the latter."""
    arr = layers if isinstance(layers, ctypes.Array) else make_layers(layers)
    return _check(lib.idx_expand_and_score_layers(
        ctypes.byref(cfg), ctypes.byref(rows), _p(candidate_blocks), cand_stride,
        ctypes.byref(sched), len(arr), arr, out_stride, _p(workspace), workspace_bytes,
        _p(stream)))


def idx_dense_masked_logits_topk(cfg, rows, max_ctx, q_values, q_scales, weights, k, sched,
                                 topk_indices, out_stride, logits_out=None, logits_stride=0,
                                 workspace=None, workspace_bytes=0, stream=None):
    return _check(lib.idx_dense_masked_logits_topk(
        ctypes.byref(cfg), ctypes.byref(rows), max_ctx, _p(q_values), _p(q_scales), _p(weights),
        ctypes.byref(k), ctypes.byref(sched), _p(topk_indices), out_stride, _p(logits_out),
        logits_stride, _p(workspace), workspace_bytes, _p(stream)))


def idx_publish_workspace_bytes(cfg: idx_config, max_rows: int, max_ctx: int) -> int:
    return lib.idx_publish_workspace_bytes(ctypes.byref(cfg), max_rows, max_ctx)


def idx_publish_candidates(cfg, rows, max_ctx, q_values, q_scales, weights, k, candidate_blocks,
                           cand_stride, logits_out=None, logits_stride=0, workspace=None,
                           workspace_bytes=0, stream=None):
    """The candidate-source layer: writes candidate_blocks [rows, >= NB] (int32 device)."""
    return _check(lib.idx_publish_candidates(
        ctypes.byref(cfg), ctypes.byref(rows), max_ctx, _p(q_values), _p(q_scales), _p(weights),
        ctypes.byref(k), _p(candidate_blocks), cand_stride, _p(logits_out), logits_stride,
        _p(workspace), workspace_bytes, _p(stream)))


def bind_publish_candidates(cfg, rows, max_ctx, q_values, q_scales, weights, k,
                            candidate_blocks, cand_stride, logits_out=None, logits_stride=0,
                            workspace=None, workspace_bytes=0, stream=None):
    vp = lambda x: ctypes.c_void_p(_p(x))
    return BoundCall(lib.idx_publish_candidates,
                     (ctypes.byref(cfg), ctypes.byref(rows), max_ctx, vp(q_values), vp(q_scales),
                      vp(weights), ctypes.byref(k), vp(candidate_blocks), cand_stride,
                      vp(logits_out), logits_stride, vp(workspace), workspace_bytes, vp(stream)),
                     (cfg, rows, k))


def idx_gather_k_workspace(cfg, k, cu_seq_lens, values_out, scales_out, max_seq_len,
                           req_table=None, stream=None):
    """Pack requests' paged K into values_out [N, D/2] / scales_out [N, D/32] (u8 device
    tensors); cu_seq_lens: int32 device tensor [num_reqs + 1]."""
    num_reqs = cu_seq_lens.numel() - 1 if cu_seq_lens is not None else 0
    _check_workspace(cfg, values_out, scales_out)
    return _check(lib.idx_gather_k_workspace(
        ctypes.byref(cfg), ctypes.byref(k), max(0, num_reqs), _p(cu_seq_lens), _p(req_table),
        max_seq_len, values_out.shape[0], _p(values_out), _p(scales_out), _p(stream)))


def _check_workspace(cfg, values_out, scales_out):
    """The library writes max_tokens = values_out.shape[0] rows of D/2 and D/32 bytes:
    both tensors must hold that many contiguous rows."""
    for t, row in ((values_out, cfg.head_dim // 2), (scales_out, cfg.head_dim // 32)):
        if not t.is_contiguous() or t.dim() != 2 or t.shape[1] * t.element_size() != row:
            raise ValueError(f"workspace tensor must be contiguous [N, {row}] bytes, got "
                             f"{tuple(t.shape)} x {t.element_size()} B")
    if scales_out.shape[0] < values_out.shape[0]:
        raise ValueError("scales_out has fewer rows than values_out")


def bind_gather_k_workspace(cfg, k, cu_seq_lens, values_out, scales_out, max_seq_len,
                            req_table=None, stream=None):
    _check_workspace(cfg, values_out, scales_out)
    vp = lambda x: ctypes.c_void_p(_p(x))
    return BoundCall(lib.idx_gather_k_workspace,
                     (ctypes.byref(cfg), ctypes.byref(k), cu_seq_lens.numel() - 1,
                      vp(cu_seq_lens), vp(req_table), max_seq_len, values_out.shape[0],
                      vp(values_out), vp(scales_out), vp(stream)), (cfg, k))


def make_workspace_kcache(values, scales, block_table) -> idx_kcache:
    """The packed workspace as a one-page cache: values u8 [N, D/2], scales u8 [N, D/32],
    block_table int32 [1, 1] holding 0."""
    return idx_kcache(values.data_ptr(), values.numel(), scales.data_ptr(), scales.numel(), 1,
                      block_table.data_ptr(), block_table.stride(0), block_table.shape[0],
                      block_table.shape[1])


def idx_measure_read(src, nbytes, sink, stream=None):
    """Reference read stream over nbytes of src (device); sink: IDX_MEASURE_WGS uint32."""
    return _check(lib.idx_measure_read(_p(src), nbytes, _p(sink), _p(stream)))


def idx_measure_mfma(iters, sink, stream=None):
    """Reference MX-FP4 MFMA loop; sink: IDX_MEASURE_WGS * 4 floats."""
    return _check(lib.idx_measure_mfma(iters, _p(sink), _p(stream)))


def idx_measure_mfma_relu(iters, sink, stream=None):
    """The MX-FP4 MFMA loop with the ReLU-weight epilogue on every product; sink as
    idx_measure_mfma, same flop count."""
    return _check(lib.idx_measure_mfma_relu(iters, _p(sink), _p(stream)))


def idx_measure_fp8_dot(q_e4m3, k_e2m1, k_scales, mode, out, stream=None):
    """16 x 16 e4m3 . (e2m1 x UE8M0) dot products into out (fp32 [16, 16], device):
    mode 0 the MX-scaled fp8 x fp4 MFMA, mode 1 the exact bf16 route of the kernels,
    mode 2 the MX-scaled fp8 x fp8 MFMA on K converted exactly to e4m3."""
    return _check(lib.idx_measure_fp8_dot(_p(q_e4m3), _p(k_e2m1), _p(k_scales), mode, _p(out),
                                          _p(stream)))


def idx_measure_mfma_flops(iters) -> int:
    return int(lib.idx_measure_mfma_flops(iters))


# ------------------------------------------------- calls bound ahead of time --

class BoundCall:
    """One C entry point with its arguments marshalled once: pointers are read from the
    tensors when the call is bound, so they must stay alive and in place.  Calling it
    costs one foreign call (a serving or benchmark loop repeats the same launch)."""

    __slots__ = ("fn", "args", "keep")

    def __init__(self, fn, args, keep):
        self.fn = fn
        self.args = tuple(args)
        self.keep = keep            # the structs the byref arguments point at

    def __call__(self) -> int:
        rc = self.fn(*self.args)
        if rc < 0:
            raise IdxError(rc, idx_last_error())
        return rc


def bind_expand_candidates(cfg, rows, k, candidate_blocks, cand_stride, sched, stream=None):
    return BoundCall(lib.idx_expand_candidates,
                     (ctypes.byref(cfg), ctypes.byref(rows), ctypes.byref(k),
                      ctypes.c_void_p(_p(candidate_blocks)), cand_stride, ctypes.byref(sched),
                      ctypes.c_void_p(_p(stream))), (cfg, rows, k, sched))


def bind_sparse_mqa_logits_topk(cfg, rows, q_values, q_scales, weights, k, sched, topk_indices,
                                out_stride, logits_out=None, workspace=None, workspace_bytes=0,
                                stream=None):
    vp = lambda x: ctypes.c_void_p(_p(x))
    return BoundCall(lib.idx_sparse_mqa_logits_topk,
                     (ctypes.byref(cfg), ctypes.byref(rows), vp(q_values), vp(q_scales),
                      vp(weights), ctypes.byref(k), ctypes.byref(sched), vp(topk_indices),
                      out_stride, vp(logits_out), vp(workspace), workspace_bytes, vp(stream)),
                     (cfg, rows, k, sched))


def bind_sparse_mqa_logits_topk_layers(cfg, rows, sched, layers, out_stride, workspace=None,
                                       workspace_bytes=0, stream=None):
    arr = layers if isinstance(layers, ctypes.Array) else make_layers(layers)
    vp = lambda x: ctypes.c_void_p(_p(x))
    return BoundCall(lib.idx_sparse_mqa_logits_topk_layers,
                     (ctypes.byref(cfg), ctypes.byref(rows), ctypes.byref(sched), len(arr), arr,
                      out_stride, vp(workspace), workspace_bytes, vp(stream)),
                     (cfg, rows, sched, arr))


def bind_expand_and_score_layers(cfg, rows, candidate_blocks, cand_stride, sched, layers,
                                 out_stride, workspace=None, workspace_bytes=0, stream=None):
    arr = layers if isinstance(layers, ctypes.Array) else make_layers(layers)
    vp = lambda x: ctypes.c_void_p(_p(x))
    return BoundCall(lib.idx_expand_and_score_layers,
                     (ctypes.byref(cfg), ctypes.byref(rows), vp(candidate_blocks), cand_stride,
                      ctypes.byref(sched), len(arr), arr, out_stride, vp(workspace),
                      workspace_bytes, vp(stream)),
                     (cfg, rows, sched, arr))


def bind_dense_masked_logits_topk(cfg, rows, max_ctx, q_values, q_scales, weights, k, sched,
                                  topk_indices, out_stride, logits_out=None, logits_stride=0,
                                  workspace=None, workspace_bytes=0, stream=None):
    vp = lambda x: ctypes.c_void_p(_p(x))
    return BoundCall(lib.idx_dense_masked_logits_topk,
                     (ctypes.byref(cfg), ctypes.byref(rows), max_ctx, vp(q_values), vp(q_scales),
                      vp(weights), ctypes.byref(k), ctypes.byref(sched), vp(topk_indices),
                      out_stride, vp(logits_out), logits_stride, vp(workspace), workspace_bytes,
                      vp(stream)), (cfg, rows, k, sched))


def event_handle(e):
    """Raw HIP event handle of a torch.cuda.Event (created on first use)."""
    if not e.cuda_event:
        e.record()
    return e.cuda_event


# ------------------------------------------------------------- torch glue ---

def _p(x):
    """Raw pointer of a torch tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr() if x.numel() else None
    if hasattr(x, "cuda_stream"):
        return x.cuda_stream
    raise TypeError(f"cannot take a pointer of {type(x)}")


def make_config(num_heads=64, head_dim=128, q_format=IDX_Q_MXFP4, page_size=64,
                candidate_block_size=64, sparse_block_kv=0, num_candidate_blocks=64,
                topk=2048, score_format=IDX_SCORE_FP32) -> idx_config:
    return idx_check_config(idx_config(num_heads, head_dim, q_format, page_size,
                                       candidate_block_size, sparse_block_kv,
                                       num_candidate_blocks, topk, score_format))


def make_kcache(pool, page_size, head_dim, block_table) -> idx_kcache:
    """K cache over one uint8 pool tensor [num_pages, page_bytes] whose pages hold the
    packed values [page_size][D/2] followed by the scales [page_size][D/32], and an
    int32 block table [num_tables, pages_per_table]."""
    page_bytes = pool.shape[1]
    k = idx_kcache(pool.data_ptr(), page_bytes, pool.data_ptr() + page_size * head_dim // 2,
                   page_bytes, pool.shape[0], block_table.data_ptr(), block_table.stride(0),
                   block_table.shape[0], block_table.shape[1])
    k._tensors = (pool, block_table)   # the struct holds their addresses: keep them alive
    return k


def make_rows(row_ke, row_ks=None, row_table=None, rows_per_request=1) -> idx_rows:
    """rows_per_request: consecutive rows of one request (next_n), a placement hint."""
    r = idx_rows(row_ke.shape[0], _p(row_ks), _p(row_ke), _p(row_table), rows_per_request)
    r._tensors = (row_ke, row_ks, row_table)   # the struct holds their addresses
    return r


class Schedule:
    """Device buffers of one step's sparse-column schedule (owned by torch)."""

    def __init__(self, cfg: idx_config, max_rows: int, device):
        import torch

        self.nsb = idx_num_sparse_blocks(cfg)
        self.sparse_indices = torch.empty((max_rows, self.nsb), dtype=torch.int32, device=device)
        self.end = torch.empty(max_rows, dtype=torch.int32, device=device)
        nbytes = max(4, idx_schedule_work_bytes(cfg, max_rows))
        self.work = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.struct = idx_schedule(self.sparse_indices.data_ptr(), self.end.data_ptr(),
                                   self.work.data_ptr(), nbytes)
