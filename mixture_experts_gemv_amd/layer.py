"""Device-resident MoE layer: uploads host weights and calls the C ABI.

Host weights come in their storage formats (fp32 ``float32``, bf16 as
``uint16`` bit patterns, Q8_0 as ``uint8`` 34-byte blocks and MXFP4 as
``uint8`` 17-byte blocks along the reduction dimension).  Q8_0 and MXFP4
tensors are split on the device into the value and scale planes the kernels
read (``moe_q8_0_split``, ``moe_mxfp4_split``).
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import (MOE_BF16, MOE_F32, MOE_MXFP4, MOE_PATH_AUTO, MOE_Q8_0, make_weights, moe_forward,
               moe_forward_fused, moe_mxfp4_split, moe_plan_create, moe_q8_0_split, moe_workspace_bytes)

_TORCH_DTYPE = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}


def upload(arr: np.ndarray, device) -> torch.Tensor:
    """Copy a host storage array to the device, keeping its bytes."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


class MoeLayer:
    """One routed-MoE layer on one GPU, with its plan and weights."""

    def __init__(self, *, hidden, num_experts, top_k, expert_inter, shared_inter=0,
                 select=0, bias_mode=0, swiglu_limit=0.0, rms_eps=0.0, x_dtype=MOE_BF16,
                 router_dtype=MOE_BF16, expert_dtype=MOE_BF16, shared_dtype=MOE_BF16,
                 max_tokens=1, path=MOE_PATH_AUTO, device="cuda"):
        self.device = torch.device(device)
        self.H, self.E, self.k = hidden, num_experts, top_k
        self.I, self.Is = expert_inter, shared_inter
        self.x_dtype, self.expert_dtype, self.router_dtype = x_dtype, expert_dtype, router_dtype
        self.shared_dtype = shared_dtype if shared_inter > 0 else expert_dtype
        self.max_tokens = max_tokens
        self.plan = moe_plan_create(hidden, num_experts, top_k, expert_inter, shared_inter,
                                    max_tokens, select, bias_mode, swiglu_limit, rms_eps,
                                    x_dtype, router_dtype, expert_dtype, self.shared_dtype, path)
        self.tensors: Dict[str, torch.Tensor] = {}
        self.weights = None

    # -- weights -------------------------------------------------------------
    def _mat(self, name: str, arr: np.ndarray, rows: int, cols: int, dtype: int):
        if dtype == MOE_Q8_0:
            blocks = upload(np.ascontiguousarray(arr).reshape(-1), self.device)
            qs = torch.empty(rows * cols, dtype=torch.int8, device=self.device)
            sc = torch.empty(rows * cols // 32, dtype=torch.int16, device=self.device)
            moe_q8_0_split(blocks, rows, cols, qs, sc)
            self.tensors[name] = qs
            self.tensors[name + "_scale"] = sc
            del blocks
        elif dtype == MOE_MXFP4:
            blocks = upload(np.ascontiguousarray(arr).reshape(-1), self.device)
            codes = torch.empty(rows * cols // 2, dtype=torch.uint8, device=self.device)
            sc = torch.empty(rows * cols // 32, dtype=torch.uint8, device=self.device)
            moe_mxfp4_split(blocks, rows, cols, codes, sc)
            self.tensors[name] = codes
            self.tensors[name + "_scale"] = sc
            del blocks
        else:
            t = upload(arr, self.device).reshape(-1)
            self.tensors[name] = t

    def load(self, router, bias, gate, up, down, shared_gate=None, shared_up=None,
             shared_down=None, router_x_scale=None) -> "MoeLayer":
        """router_x_scale: the router's per-element input scale (bf16 bits
        [H]) or None."""
        H, E, I, Is = self.H, self.E, self.I, self.Is
        self.tensors.clear()
        if self.router_dtype == MOE_Q8_0:
            self._mat("router", router, E, H, MOE_Q8_0)
        else:
            self.tensors["router"] = upload(router, self.device).reshape(-1)
        if router_x_scale is not None:
            self.tensors["router_x_scale"] = upload(np.asarray(router_x_scale, np.uint16), self.device)
        if bias is not None:
            self.tensors["bias"] = upload(np.asarray(bias, np.float32), self.device)
        self._mat("gate", gate, E * I, H, self.expert_dtype)
        self._mat("up", up, E * I, H, self.expert_dtype)
        self._mat("down", down, E * H, I, self.expert_dtype)
        if Is > 0:
            self._mat("shared_gate", shared_gate, Is, H, self.shared_dtype)
            self._mat("shared_up", shared_up, Is, H, self.shared_dtype)
            self._mat("shared_down", shared_down, H, Is, self.shared_dtype)
        torch.cuda.synchronize(self.device)
        self.weights = make_weights(**self.tensors)
        return self

    def load_tensors(self, tensors: Dict[str, torch.Tensor]) -> "MoeLayer":
        """Use device tensors already in the planes' layout (names as moe_weights)."""
        self.tensors = dict(tensors)
        self.weights = make_weights(**self.tensors)
        return self

    # -- calls ---------------------------------------------------------------
    def workspace(self, M: int) -> torch.Tensor:
        n = max(256, moe_workspace_bytes(self.plan, M))
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def x_tensor(self, x: np.ndarray) -> torch.Tensor:
        return upload(x, self.device)

    def forward(self, x: torch.Tensor, ws: Optional[torch.Tensor] = None, y=None, ids=None,
                w=None, counts=None, stream=None) -> torch.Tensor:
        M = x.shape[0]
        if ws is None:
            ws = self.workspace(M)
        if y is None:
            y = torch.empty(M, self.H, dtype=torch.float32, device=self.device)
        moe_forward(self.plan, x, self.weights, M, y, ids, w, counts, ws, stream)
        return y

    def forward_fused(self, x: torch.Tensor, norm_weight=None, residual=None, ws=None, y=None,
                      ids=None, w=None, counts=None, stream=None) -> torch.Tensor:
        """y = residual + layer(rms_norm(x) * norm_weight) (moe_forward_fused)."""
        M = x.shape[0]
        if ws is None:
            ws = self.workspace(M)
        if y is None:
            y = torch.empty(M, self.H, dtype=torch.float32, device=self.device)
        moe_forward_fused(self.plan, x, norm_weight, residual, self.weights, M, y, ids, w, counts, ws,
                          stream)
        return y
