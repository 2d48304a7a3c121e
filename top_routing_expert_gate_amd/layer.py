"""A small convenience wrapper around ``moe_forward``: holds the parameter
tensors (on the GPU), the descriptor and a cached workspace, and allocates
the output.  Marshalling and memory only -- every step of the layer runs in
libmoe's HIP kernels."""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B

_DT = {torch.float32: B.MOE_F32, torch.bfloat16: B.MOE_BF16}


class MoELayer:
    """Sparse MoE FFN forward on one GPU.

    ``params`` maps the ``moe_weights`` member names (w_router, router_bias,
    sel_bias, w_act, w_lin, w_down, b_act, b_down, ws_*, bs_*) to CUDA
    tensors in the nn.Linear layouts documented in include/moe.h.
    """

    _SCORES = {"softmax": B.MOE_SCORE_SOFTMAX, "sigmoid": B.MOE_SCORE_SIGMOID,
               "softmax_all": B.MOE_SCORE_SOFTMAX_ALL}
    _EXPERTS = {"swiglu": B.MOE_EXPERT_SWIGLU, "silu_mlp": B.MOE_EXPERT_SILU_MLP,
                "gelu_mlp": B.MOE_EXPERT_GELU_MLP}
    _DROPS = {"zero": B.MOE_DROP_ZERO, "residual": B.MOE_DROP_RESIDUAL}

    def __init__(self, params: dict, *, k: int, score: str = "softmax",
                 expert: str = "swiglu", capacity: int = -1, drop: str = "zero"):
        self.params = {n: t for n, t in params.items() if t is not None}
        w_act = self.params["w_act"]
        self.E, self.d_ff, self.d_model = w_act.shape
        self.dtype = w_act.dtype
        self.k = k
        self.score_fn = self._SCORES[score]
        self.expert_kind = self._EXPERTS[expert]
        self.drop_policy = self._DROPS[drop]
        self.n_shared = 1 if "ws_act" in self.params else 0
        self.capacity = capacity
        self.weights = B.make_weights(**self.params)
        self._ws: Optional[torch.Tensor] = None

    def desc(self, T: int) -> B.MoeDesc:
        return B.make_desc(T, self.d_model, self.d_ff, self.E, self.k, _DT[self.dtype],
                           self.score_fn, self.expert_kind, self.n_shared, self.capacity,
                           drop_policy=self.drop_policy)

    def workspace(self, T: int) -> torch.Tensor:
        n = B.moe_workspace_size(self.desc(T))
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.params["w_act"].device)
        return self._ws

    def __call__(self, x: torch.Tensor, aux: Optional[B.MoeForwardAux] = None) -> torch.Tensor:
        shape = x.shape
        flat = x.reshape(-1, self.d_model).contiguous()  # rows = flattened tokens
        out = torch.empty_like(flat)
        d = self.desc(flat.shape[0])
        B.moe_forward(d, self.weights, flat, out, aux, self.workspace(flat.shape[0]))
        return out.reshape(shape)
