"""Device-resident layer: uploads a workload to HIP memory and calls the C ABI.

Only allocation and marshalling happen here (torch is used for device memory
and streams); every step of the computation runs in ``libkt_rawint4.so``.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import _lib
from .workloads import LORA_NAMES, LayerConfig, Weights


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 tensor on ``device``."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceLayer:
    """One MoE layer in device memory.  ``base_only=True`` uploads no LoRA and
    passes NULL for all six LoRA pointers: such a layer serves only the
    inference forward of the frozen base."""

    def __init__(self, cfg: LayerConfig, weights: Weights, device="cuda", lora: Optional[Dict[str, np.ndarray]] = None,
                 base_only: bool = False):
        self.cfg = cfg
        self.device = torch.device(device)
        dev = self.device
        self.gate_packed = torch.from_numpy(weights.gate_packed).to(dev)
        self.up_packed = torch.from_numpy(weights.up_packed).to(dev)
        self.down_packed = torch.from_numpy(weights.down_packed).to(dev)
        self.gate_scale = bf16_tensor(weights.gate_scale, dev)
        self.up_scale = bf16_tensor(weights.up_scale, dev)
        self.down_scale = bf16_tensor(weights.down_scale, dev)
        if base_only:
            self.lora = {n: None for n in LORA_NAMES}
        else:
            src = weights.lora if lora is None else lora
            self.lora = {n: torch.from_numpy(np.ascontiguousarray(src[n], dtype=np.float32)).to(dev)
                         for n in LORA_NAMES}
        self.layer = _lib.make_layer(cfg.num_experts, cfg.top_k, cfg.hidden, cfg.intermediate, cfg.rank, cfg.alpha,
                                     cfg.swiglu_limit, self.gate_packed, self.up_packed, self.down_packed,
                                     self.gate_scale, self.up_scale, self.down_scale,
                                     *(self.lora[n] for n in LORA_NAMES), weight_format=cfg.weight_format)

    def workspace(self, qlen: int) -> torch.Tensor:
        n = _lib.kt_rawint4_moe_workspace_bytes(self.layer, qlen)
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def infer_workspace(self, qlen: int) -> torch.Tensor:
        n = _lib.kt_rawint4_moe_infer_workspace_bytes(self.layer, qlen)
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def grad_buffers(self, fill: Optional[float] = None) -> Dict[str, torch.Tensor]:
        shapes = self.cfg.lora_shapes()
        if fill is None:
            return {n: torch.empty(shapes[n], dtype=torch.float32, device=self.device) for n in LORA_NAMES}
        return {n: torch.full(shapes[n], fill, dtype=torch.float32, device=self.device) for n in LORA_NAMES}

    def forward(self, inputs, expert_ids, route_weights, workspace, output=None, stream=None) -> torch.Tensor:
        qlen = inputs.shape[0]
        if output is None:
            output = torch.empty((qlen, self.cfg.hidden), dtype=torch.bfloat16, device=self.device)
        _lib.kt_rawint4_moe_fwd(self.layer, qlen, inputs, expert_ids, route_weights, output, workspace, stream)
        return output

    def infer(self, inputs, expert_ids, route_weights, workspace, output=None, stream=None) -> torch.Tensor:
        """Forward that keeps nothing for a backward (the output equals forward()'s)."""
        qlen = inputs.shape[0]
        if output is None:
            output = torch.empty((qlen, self.cfg.hidden), dtype=torch.bfloat16, device=self.device)
        _lib.kt_rawint4_moe_infer(self.layer, qlen, inputs, expert_ids, route_weights, output, workspace, stream)
        return output

    def backward(self, inputs, expert_ids, route_weights, grad_output, workspace, grads, accumulate=False,
                 grad_scale=1.0, grad_input=None, grad_route=None, stream=None, recompute=False):
        """recompute=True: the workspace need not hold this call's forward (it is rerun first)."""
        qlen = inputs.shape[0]
        if grad_input is None:
            grad_input = torch.empty((qlen, self.cfg.hidden), dtype=torch.bfloat16, device=self.device)
        fn = _lib.kt_rawint4_moe_bwd_recompute if recompute else _lib.kt_rawint4_moe_bwd
        fn(self.layer, qlen, inputs, expert_ids, route_weights, grad_output, grad_input, grad_route,
           *(grads[n] for n in LORA_NAMES), accumulate, grad_scale, workspace, stream)
        return grad_input, grad_route

    def saved_preactivations(self, qlen, workspace, stream=None):
        """Gate and up pre-activations of the latest forward in ``workspace``, [qlen, k, I] fp32 each."""
        shape = (qlen, self.cfg.top_k, self.cfg.intermediate)
        gate = torch.empty(shape, dtype=torch.float32, device=self.device)
        up = torch.empty(shape, dtype=torch.float32, device=self.device)
        _lib.kt_rawint4_moe_saved_preactivations(self.layer, qlen, workspace, gate, up, stream)
        return gate, up


class DeviceBatch:
    def __init__(self, batch, device="cuda"):
        dev = torch.device(device)
        self.inputs = bf16_tensor(batch.inputs, dev)
        self.expert_ids = torch.from_numpy(np.ascontiguousarray(batch.expert_ids, dtype=np.int64)).to(dev)
        self.route_weights = torch.from_numpy(np.ascontiguousarray(batch.route_weights, dtype=np.float32)).to(dev)
        self.grad_output = bf16_tensor(batch.grad_output, dev)
        self.qlen = self.inputs.shape[0]
