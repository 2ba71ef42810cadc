"""Copy a generated case to a torch device (input plumbing: no arithmetic).

The K page pool is allocated zero-filled on the device and only the pages that
hold contents are copied in, so multi-GB fragmented pools cost only the bytes
that are actually drawn.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class DeviceLayer:
    pool: object                 # uint8 [num_pages, page_bytes]
    weights: object              # float32 [R, H]
    q_values: object = None      # uint8 [R, H, D/2]
    q_scales: object = None      # uint8 [R, H, D/32]
    q_fp8: object = None         # uint8 [R, H, D]
    q_rowscale: object = None    # float32 [R]
    weights_bf16: object = None  # int16 [R, H]: the weights' bf16 codes

    def w(self, score_format: str = "fp32"):
        """The weights argument for the given scoring format."""
        return self.weights_bf16 if score_format == "bf16" else self.weights

    def q(self, q_format: str):
        """(q_values, q_scales) arguments for the given query format."""
        if q_format == "mxfp4":
            return self.q_values, self.q_scales
        return self.q_fp8, self.q_rowscale


@dataclass
class DeviceCase:
    row_ks: object
    row_ke: object
    row_table: object
    block_table: object
    candidate_blocks: object
    layers: list = field(default_factory=list)


def _t(a, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def layer_to_device(spec, L, device):
    import torch

    pool = torch.zeros((L.num_pages, spec.page_bytes), dtype=torch.uint8, device=device)
    if len(L.filled_pages):
        idx = torch.from_numpy(L.filled_pages.astype(np.int64)).to(device)
        pool.index_copy_(0, idx, _t(L.filled_data, device))
    return DeviceLayer(
        pool=pool, weights=_t(L.weights.astype(np.float32), device),
        q_values=None if L.q_values is None else _t(L.q_values, device),
        q_scales=None if L.q_scales is None else _t(L.q_scales, device),
        q_fp8=None if L.q_fp8 is None else _t(L.q_fp8, device),
        q_rowscale=None if L.q_rowscale is None else _t(L.q_rowscale.astype(np.float32), device),
        weights_bf16=_t(L.weights_bf16.view(np.int16), device))


def to_device(case, device, layers=None) -> DeviceCase:
    layers = range(len(case.layers)) if layers is None else layers
    return DeviceCase(
        row_ks=_t(case.row_ks.astype(np.int32), device),
        row_ke=_t(case.row_ke.astype(np.int32), device),
        row_table=_t(case.row_table.astype(np.int32), device),
        block_table=_t(case.block_table.astype(np.int32), device),
        candidate_blocks=_t(case.candidate_blocks.astype(np.int32), device),
        layers=[layer_to_device(case.spec, case.layers[i], device) for i in layers])
