"""The Hyper-Connection mixer around the attention block (four residual
streams), as device tensors over libckv's ``ckv_hc_pre`` / ``ckv_hc_post``.
Argument marshalling only: the split, the Sinkhorn normalisation and both
stream mixes run in the library's HIP kernels."""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib as L


class HCMixer:
    def __init__(self, hidden: int, act_fmt: str = "bf16", sinkhorn_iters: int = 20, eps: float = 1e-6,
                 device: str = "cuda"):
        self.desc = L.HcDesc(hidden=hidden, n_hc=4, sinkhorn_iters=sinkhorn_iters, eps=eps,
                             act_fmt=L.FMT[act_fmt])
        rc = L.hc_validate(self.desc)
        if rc:
            raise L.CkvError(rc, "ckv_hc_validate")
        self.hidden, self.act_fmt, self.device = hidden, act_fmt, torch.device(device)
        self.dtype = torch.float32 if act_fmt == "f32" else torch.bfloat16

    def _stream(self):
        return torch.cuda.current_stream(self.device).cuda_stream

    def pre(self, mix: torch.Tensor, h: torch.Tensor, x: Optional[torch.Tensor] = None,
            coef: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
        """mix [T, 24] float32, h [T, 4, hidden] -> (x [T, hidden], coef [T, 24])."""
        T = mix.shape[0]
        x = torch.empty((T, self.hidden), dtype=self.dtype, device=self.device) if x is None else x
        coef = torch.empty((T, 24), dtype=torch.float32, device=self.device) if coef is None else coef
        rc = L.hc_pre(self.desc, mix.data_ptr(), h.data_ptr(), T, x.data_ptr(), coef.data_ptr(), self._stream())
        if rc:
            raise L.CkvError(rc, "ckv_hc_pre")
        return x, coef

    def post(self, coef: torch.Tensor, h: torch.Tensor, y: torch.Tensor,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """coef [T, 24], h [T, 4, hidden], y [T, hidden] -> h_out [T, 4, hidden]."""
        T = coef.shape[0]
        out = torch.empty_like(h) if out is None else out
        rc = L.hc_post(self.desc, coef.data_ptr(), h.data_ptr(), y.data_ptr(), T, out.data_ptr(), self._stream())
        if rc:
            raise L.CkvError(rc, "ckv_hc_post")
        return out
