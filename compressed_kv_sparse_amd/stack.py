"""Decode driver for a stack of compressed-KV attention layers.

The layer schedule follows "ds4.c を読み解く (#3)", section 1:

* Flash: the first two layers keep only the 128-token sliding window
  (ratio 0); from layer 2 on, even layers compress at ratio 4 (c4a, with the
  indexer and top-k) and odd layers at ratio 128 (c128a);
* Pro: the first two layers are c128a, then the same alternation.

Compressed layers rotate with the compressed-row RoPE base, window-only
layers with the normal base (same page, section 8).  Each layer owns its
caches, weights and workspace; a step runs every layer's three calls in
order on the current stream, so the whole stack can be captured as one HIP
graph.  No work is shared between layers: the stack is 43 independent
single-layer steps, as the attention layers of the model are between their
(absent) feed-forward blocks.

With ``paged`` the compressed rows of every layer live in pages of pools that
all layers share, one pool per page size ("vLLM DeepSeek V4", KV cache memory
management: three page sizes for the whole stack -- c4a K=V pages, c4a indexer
pages, c128a K=V pages), each layer reaching its pages through its own block
table.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import torch

from . import _lib as L
from .layer import DeviceLayer
from .paged import BLOCK_TOKENS, PagePools

SCHEDULES = ("flash", "pro")


def layer_ratio(il: int, schedule: str = "flash") -> int:
    """Compression ratio of layer ``il`` (0 = sliding window only)."""
    if schedule not in SCHEDULES:
        raise ValueError(f"unknown schedule {schedule!r}")
    if il < 2:
        return 0 if schedule == "flash" else 128
    return 4 if il % 2 == 0 else 128


@dataclass
class StackShape:
    n_layers: int = 43
    schedule: str = "flash"
    batch: int = 16
    n_ctx: int = 131072            # capacity: compressed rows n_ctx / ratio per sequence
    hidden: int = 4096
    head_dim: int = 512
    n_heads: int = 64
    idx_heads: int = 64
    idx_dim: int = 128
    top_k: int = 512
    kv_fmt: str = "e4m3"
    idx_fmt: str = "bf16"
    rope_base_raw: float = 10000.0
    rope_base_comp: float = 160000.0
    norm_eps: float = 1e-6
    paged: bool = False            # compressed rows in shared page pools (block tables)


class DeviceStack:
    """One DeviceLayer per layer of the schedule."""

    def __init__(self, shape: StackShape, device: str = "cuda"):
        self.shape = s = shape
        self.ratios = [layer_ratio(il, s.schedule) for il in range(s.n_layers)]
        self.layers: List[DeviceLayer] = []
        self.pools = None
        if s.paged:   # every layer's whole capacity, in pages of the shared pools
            per_seq = s.n_ctx // BLOCK_TOKENS
            self.pools = PagePools(
                kv_row_bytes=L.row_bytes(L.FMT[s.kv_fmt], s.head_dim, 64),
                idx_row_bytes=L.idx_row_bytes(L.FMT[s.idx_fmt], s.idx_dim),
                pages_c4a=self.ratios.count(4) * s.batch * per_seq,
                pages_c128a=self.ratios.count(128) * s.batch * per_seq, device=device)
        for r in self.ratios:
            ci = r == 4
            self.layers.append(DeviceLayer(
                ratio=r, hidden=s.hidden, head_dim=s.head_dim, n_heads=s.n_heads, batch=s.batch,
                idx_heads=s.idx_heads if ci else 0, idx_dim=s.idx_dim if ci else 0,
                top_k=s.top_k if ci else 0, comp_cap=(s.n_ctx // r) if r else 0, kv_fmt=s.kv_fmt,
                idx_fmt=s.idx_fmt, rope_base=s.rope_base_comp if r else s.rope_base_raw,
                norm_eps=s.norm_eps, pages=self.pools, device=device))

    def __len__(self) -> int:
        return len(self.layers)

    def decode(self, inputs: List[Dict[str, Optional[torch.Tensor]]],
               outs: Optional[List[torch.Tensor]] = None,
               topks: Optional[List[Optional[torch.Tensor]]] = None) -> List[torch.Tensor]:
        """One decode step of every layer.  ``inputs[il]`` holds the device
        tensors x, u, q, qI, w, pos of layer il (qI and w None off c4a layers)."""
        if len(inputs) != len(self.layers):
            raise ValueError(f"{len(inputs)} input sets for {len(self.layers)} layers")
        res = []
        for il, (dl, a) in enumerate(zip(self.layers, inputs)):
            o = outs[il] if outs is not None else None
            tk = topks[il] if topks is not None else None
            o, _ = dl.decode_step(a["x"], a["u"], a["q"], a.get("qI"), a.get("w"), a["pos"], out=o, topk=tk)
            res.append(o)
        return res

    def buffers(self):
        """Preallocated outputs and top-k lists (for graph capture)."""
        outs = [dl.new_out(dl.batch) for dl in self.layers]
        topks = [torch.empty((dl.batch, dl.k), dtype=torch.int32, device=dl.device) if dl.ratio == 4 else None
                 for dl in self.layers]
        return outs, topks
