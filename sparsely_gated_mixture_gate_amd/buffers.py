"""Device-memory plumbing for the MoE library: torch tensors for inputs,
outputs and the workspace. Allocation and copies only; every step of the layer
runs in the library's kernels."""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (MOE_OP_DISPATCH, MOE_OP_EXPERT_FFN, MOE_OP_FORWARD, MOE_OP_ROUTE, moe_max_rows, moe_params,
               moe_workspace_size)


def to_device(a, device="cuda"):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_numpy(t):
    """device tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def workspace(p: moe_params, op: int, device="cuda") -> torch.Tensor:
    n = max(moe_workspace_size(p, op), 256)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def elt_dtype(p: moe_params):
    return torch.bfloat16 if p.dtype == 1 else torch.float32


@dataclass
class ForwardBuffers:
    y: torch.Tensor
    aux: torch.Tensor
    topk_idx: torch.Tensor
    topk_gate: torch.Tensor
    counts_routed: torch.Tensor
    counts_kept: torch.Tensor
    slot_dest: torch.Tensor
    ws: torch.Tensor

    @classmethod
    def alloc(cls, p: moe_params, device="cuda") -> "ForwardBuffers":
        T, k, E, d = p.T, p.k, p.E, p.d_model
        return cls(
            y=torch.empty((T, d), dtype=elt_dtype(p), device=device),
            aux=torch.empty(4, dtype=torch.float32, device=device),
            topk_idx=torch.empty((T, k), dtype=torch.int32, device=device),
            topk_gate=torch.empty((T, k), dtype=torch.float32, device=device),
            counts_routed=torch.empty(E, dtype=torch.int32, device=device),
            counts_kept=torch.empty(E, dtype=torch.int32, device=device),
            slot_dest=torch.empty((T, k), dtype=torch.int32, device=device),
            ws=workspace(p, MOE_OP_FORWARD, device),
        )


@dataclass
class StepBuffers:
    """Outputs of the four step entry points (route, dispatch, expert FFN, combine)."""

    topk_idx: torch.Tensor
    topk_gate: torch.Tensor
    counts_routed: torch.Tensor
    aux: torch.Tensor
    logits: torch.Tensor
    counts_kept: torch.Tensor
    offsets: torch.Tensor
    slot_dest: torch.Tensor
    row_src: torch.Tensor
    x_perm: torch.Tensor
    y_perm: torch.Tensor
    y: torch.Tensor
    ws_route: torch.Tensor
    ws_dispatch: torch.Tensor
    ws_ffn: torch.Tensor

    @classmethod
    def alloc(cls, p: moe_params, device="cuda") -> "StepBuffers":
        T, k, E, d = p.T, p.k, p.E, p.d_model
        R = max(moe_max_rows(p), 1)
        dt = elt_dtype(p)
        return cls(
            topk_idx=torch.empty((T, k), dtype=torch.int32, device=device),
            topk_gate=torch.empty((T, k), dtype=torch.float32, device=device),
            counts_routed=torch.empty(E, dtype=torch.int32, device=device),
            aux=torch.empty(4, dtype=torch.float32, device=device),
            logits=torch.empty((T, E), dtype=torch.float32, device=device),
            counts_kept=torch.empty(E, dtype=torch.int32, device=device),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=device),
            slot_dest=torch.empty((T, k), dtype=torch.int32, device=device),
            row_src=torch.full((R,), -1, dtype=torch.int32, device=device),
            x_perm=torch.zeros((R, d), dtype=dt, device=device),
            y_perm=torch.zeros((R, d), dtype=dt, device=device),
            y=torch.empty((T, d), dtype=dt, device=device),
            ws_route=workspace(p, MOE_OP_ROUTE, device),
            ws_dispatch=workspace(p, MOE_OP_DISPATCH, device),
            ws_ffn=workspace(p, MOE_OP_EXPERT_FFN, device),
        )
