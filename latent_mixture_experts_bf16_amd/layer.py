"""Put one layer's weights in device memory and drive it through the C ABI.

PyTorch only allocates device memory and provides the stream; every computation runs in
the library's HIP kernels (binding.py). Host arrays follow the layouts of
include/moe_latent.h: 16-bit values as uint16 bit patterns, codes as uint32 words.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import binding as B

_TORCH_VIEW = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32,
               np.dtype(np.float32): np.float32, np.dtype(np.int32): np.int32}


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(_TORCH_VIEW[a.dtype])).to(device)


def config_of(dims, max_rows: int) -> B.moe_latent_config:
    c = B.moe_latent_config()
    c.hidden, c.latent, c.n_experts = dims.hidden, dims.latent, dims.n_experts
    c.n_group, c.topk_group, c.top_k = dims.n_group, dims.topk_group, dims.top_k
    c.expert_inter, c.shared_inter, c.group_size = dims.expert_inter, dims.shared_inter, dims.group_size
    c.act_dtype = B.MOE_DT_F16 if dims.act_dtype == 2 else B.MOE_DT_BF16
    c.router_dtype = B.MOE_DT_F32 if dims.router_dtype == 3 else B.MOE_DT_BF16
    c.activation = B.MOE_ACT_RELU2
    c.has_bias = int(dims.has_bias)
    c.norm_topk = int(dims.norm_topk)
    c.max_rows = max_rows
    c.routed_scaling = dims.routed_scaling
    c.quant_bits = dims.quant_bits
    return c


_DT = {"gate_w": None, "corr_bias": B.MOE_DT_F32, "fc1_w": B.MOE_DT_BF16, "fc2_w": B.MOE_DT_BF16,
       "up_q": B.MOE_DT_U32, "up_scales": B.MOE_DT_BF16, "up_biases": B.MOE_DT_BF16,
       "down_q": B.MOE_DT_U32, "down_scales": B.MOE_DT_BF16, "down_biases": B.MOE_DT_BF16,
       "shared_up": B.MOE_DT_BF16, "shared_down": B.MOE_DT_BF16}


def weights_of(dims, dev: Dict[str, torch.Tensor]) -> B.moe_latent_weights:
    w = B.moe_latent_weights()
    for name in B.WEIGHT_FIELDS:
        t = dev.get(name)
        if t is None:
            continue
        dt = _DT[name]
        if dt is None:
            dt = B.MOE_DT_F32 if dims.router_dtype == 3 else B.MOE_DT_BF16
        setattr(w, name, B.make_tensor(t.data_ptr(), dt, list(t.shape), list(t.stride())))
    return w


class DeviceLayer:
    """One layer instance resident on the GPU, with its C handle."""

    def __init__(self, dims, arrays: Dict[str, np.ndarray], max_rows: int, stream: int = 0,
                 variant: Optional[int] = None):
        self.dims = dims
        self.max_rows = max_rows
        self.dev = {k: to_device(v) for k, v in arrays.items() if k != "x"}
        self.cfg = config_of(dims, max_rows)
        self.w = weights_of(dims, self.dev)
        self.handle = B.moe_latent_create(self.cfg, self.w, stream)
        if variant is not None:
            B.moe_latent_set_variant(self.handle, variant)

    def forward(self, x: torch.Tensor, out: torch.Tensor, rows: Optional[int] = None) -> None:
        rows = x.shape[0] if rows is None else rows
        B.moe_latent_forward(self.handle, rows, x.data_ptr(), out.data_ptr())

    def prefill(self, x: torch.Tensor, out: torch.Tensor, rows: Optional[int] = None) -> None:
        rows = x.shape[0] if rows is None else rows
        B.moe_latent_prefill(self.handle, rows, x.data_ptr(), out.data_ptr())

    def routing(self, rows: int):
        idx = torch.empty((rows, self.dims.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((rows, self.dims.top_k), dtype=torch.float32, device="cuda")
        B.moe_latent_get_routing(self.handle, idx.data_ptr(), w.data_ptr())
        torch.cuda.synchronize()
        return idx.cpu().numpy(), w.cpu().numpy()

    def stage(self, name: str, rows: int) -> np.ndarray:
        d = self.dims
        D = d.latent or d.hidden
        sizes = {"logits": d.n_experts, "latent": D, "expert_act": d.top_k * d.expert_inter,
                 "expert_out": d.top_k * D, "combine": D, "shared_act": d.shared_inter,
                 "shared_out": d.hidden}
        n = rows * sizes[name]
        f32 = name == "logits" and d.router_dtype == 3
        t = torch.empty(n, dtype=torch.float32 if f32 else torch.int16, device="cuda")
        B.moe_latent_read_stage(self.handle, B.STAGE[name], t.data_ptr(), n * (4 if f32 else 2))
        torch.cuda.synchronize()
        a = t.cpu().numpy()
        return a if f32 else a.view(np.uint16).reshape(rows, -1)

    def status(self) -> None:
        B.moe_latent_status(self.handle)

    def close(self) -> None:
        if self.handle:
            B.moe_latent_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
