"""Device-memory holder for one compressed-KV attention layer.

PyTorch supplies device memory and the stream; every step of the layer runs
in libckv's HIP kernels through the C ABI (``_lib``).  A DeviceLayer owns the
layer's cache tensors, its weights and a workspace, and exposes the three
calls per step (compress_append -> indexer_topk -> sparse_swa_attn) for
decode and chunked prefill.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np
import torch

from . import _lib as L
from .paged import BlockTable, PagePools, rows_per_block


def _dev(a, device) -> torch.Tensor:
    """numpy array / tensor -> contiguous device tensor holding the same bytes."""
    if isinstance(a, torch.Tensor):
        return a.to(device).contiguous()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceLayer:
    def __init__(self, *, ratio: int, hidden: int, head_dim: int, n_heads: int, batch: int,
                 idx_heads: int = 0, idx_dim: int = 0, top_k: int = 0, comp_cap: int = 0,
                 kv_fmt: str = "bf16", idx_fmt: str = "bf16", act_fmt: str = "bf16", w_fmt: str = "bf16",
                 rope_base: float = 160000.0, norm_eps: float = 1e-6, softmax_scale: float = 0.0,
                 flags: int = 0, n_rot: int = 64, swa: int = 128, max_chunk: int = 0,
                 rope_base_comp: float = 0.0, track_tokens: bool = True, pages: Optional[PagePools] = None,
                 device: str = "cuda"):
        """pages: page pools for a paged compressed cache (256-position
        blocks through a block table; ratio 4 / 128 only), else contiguous
        [batch, comp_cap] rows."""
        self.device = torch.device(device)
        self.desc = L.LayerDesc(ratio=ratio, hidden=hidden, head_dim=head_dim, n_rot=n_rot, n_heads=n_heads,
                                swa=swa, idx_heads=idx_heads, idx_dim=idx_dim, top_k=top_k, comp_cap=comp_cap,
                                batch=batch, kv_fmt=L.FMT[kv_fmt], idx_fmt=L.FMT[idx_fmt],
                                act_fmt=L.FMT[act_fmt], w_fmt=L.FMT[w_fmt], flags=flags,
                                rope_base=rope_base, norm_eps=norm_eps, softmax_scale=softmax_scale,
                                rope_base_comp=rope_base_comp or 0.0)
        rc = L.validate(self.desc)
        if rc:
            raise L.CkvError(rc, "ckv_validate")
        self.ratio, self.batch, self.d, self.H = ratio, batch, head_dim, n_heads
        self.HI, self.DI, self.k, self.cap, self.swa = idx_heads, idx_dim, top_k, comp_cap, swa
        self.act_fmt, self.kv_fmt, self.idx_fmt = act_fmt, kv_fmt, idx_fmt
        self.rb = L.row_bytes(L.FMT[kv_fmt], head_dim, n_rot)
        W = {4: 8, 128: 128}.get(ratio, 0)
        dev = self.device
        z8 = lambda *s: torch.zeros(s, dtype=torch.uint8, device=dev)
        zf = lambda *s: torch.zeros(s, dtype=torch.float32, device=dev)
        self.raw = z8(batch, swa, self.rb)
        self.irb = L.idx_row_bytes(L.FMT[idx_fmt], idx_dim) if ratio == 4 else 0
        self.paged = pages is not None and ratio != 0
        self.table = None
        if self.paged:   # page pools shared with other layers; rows reach them through the block table
            if pages.kv_row_bytes != self.rb or (ratio == 4 and pages.idx_row_bytes != self.irb):
                raise ValueError("the page pools' row sizes do not match this layer")
            self.rpb = rows_per_block(ratio)
            self.comp = pages.kv_pool(ratio)
            self.idx = pages.idx_pool() if ratio == 4 else None
            self.table = BlockTable(pages.free[ratio], batch, comp_cap // self.rpb, device=dev)
        else:
            self.comp = z8(batch, comp_cap, self.rb) if ratio else None
            if ratio == 4 and idx_fmt == "fp4":   # 68-byte MXFP4 records
                self.idx = z8(batch, comp_cap, self.irb)
            else:
                idt = torch.float32 if idx_fmt == "f32" else torch.int16
                self.idx = torch.zeros((batch, comp_cap, idx_dim), dtype=idt, device=dev) if ratio == 4 else None
        # a ring slot holds every compressor lane of its token (two on two-lane c4a layers)
        self.lanes = 2 if ratio == 4 and flags & L.CKV_FLAG_TWO_LANE else 1
        self.st_kv = zf(batch, W, self.lanes * head_dim) if ratio else None
        self.st_sc = zf(batch, W, self.lanes * head_dim) if ratio else None
        self.ist_kv = zf(batch, 8, self.lanes * idx_dim) if ratio == 4 else None
        self.ist_sc = zf(batch, 8, self.lanes * idx_dim) if ratio == 4 else None
        self.max_chunk = max_chunk
        self.stage = z8(max_chunk + swa - 1, self.rb) if max_chunk else None
        self.status = torch.zeros(batch, dtype=torch.int32, device=dev)
        # tokens stored per sequence (its next position); the library checks
        # every appended position against it when tracking is on
        self.n_tokens = torch.zeros(batch, dtype=torch.int32, device=dev)
        self._host_tokens = None
        self.cache = L.LayerCache(
            raw=self.raw.data_ptr(), comp=self._ptr(self.comp), idx=self._ptr(self.idx),
            st_kv=self._ptr(self.st_kv), st_sc=self._ptr(self.st_sc), ist_kv=self._ptr(self.ist_kv),
            ist_sc=self._ptr(self.ist_sc), raw_stage=self._ptr(self.stage),
            stage_rows=(max_chunk + swa - 1) if max_chunk else 0, status=self.status.data_ptr(),
            n_tokens=self.n_tokens.data_ptr() if track_tokens else None, n_tokens_host=None,
            block_table=self.table.dev.data_ptr() if self.paged else None,
            n_pages=pages.n_pages(ratio) if self.paged else 0)
        self.weights = None
        self._wt = {}
        nb = max(L.workspace_bytes(self.desc, L.CKV_MODE_DECODE, batch),
                 L.workspace_bytes(self.desc, L.CKV_MODE_PREFILL, max_chunk) if max_chunk else 0)
        self.ws = torch.zeros(nb, dtype=torch.uint8, device=dev)   # the sync region must start zeroed
        self.ws_bytes = nb

    @staticmethod
    def _ptr(t: Optional[torch.Tensor]):
        return None if t is None else t.data_ptr()

    # -------------------------------------------------------------- loading
    def set_weights(self, wkv=None, wgate=None, ape=None, gamma=None, idx_wkv=None, idx_wgate=None,
                    idx_ape=None, idx_gamma=None) -> None:
        names = dict(wkv=wkv, wgate=wgate, ape=ape, gamma=gamma, idx_wkv=idx_wkv, idx_wgate=idx_wgate,
                     idx_ape=idx_ape, idx_gamma=idx_gamma)
        self._wt = {k: (_dev(v, self.device) if v is not None else None) for k, v in names.items()}
        self.weights = L.LayerWeights(**{k: self._ptr(v) for k, v in self._wt.items()})

    def set_host_tokens(self, counts) -> None:
        """Give the library a host mirror of the token counts (a numpy int32
        array the caller keeps up to date; None removes it): prefill calls whose
        pos0 differs from it then fail with CKV_E_SEQUENCE before any work."""
        if counts is None:
            self._host_tokens = None
            self.cache.n_tokens_host = None
            return
        arr = np.ascontiguousarray(counts, dtype=np.int32)
        if arr.shape != (self.batch,):
            raise ValueError(f"host token counts must have shape ({self.batch},)")
        self._host_tokens = arr
        self.cache.n_tokens_host = arr.ctypes.data

    def load_cache(self, raw=None, comp=None, idx=None, st_kv=None, st_sc=None, ist_kv=None,
                   ist_sc=None, n_tokens=None) -> None:
        """Copy cache contents in; comp / idx in the contiguous [batch,
        comp_cap, ...] shape (a paged layer maps every block first and
        scatters the rows into its pages)."""
        for name, a in (("raw", raw), ("comp", comp), ("idx", idx), ("st_kv", st_kv), ("st_sc", st_sc),
                        ("ist_kv", ist_kv), ("ist_sc", ist_sc), ("n_tokens", n_tokens)):
            if name == "n_tokens" and a is not None:
                a = np.asarray(a, dtype=np.int32)
            if a is None:
                continue
            if self.paged and name in ("comp", "idx"):
                self._scatter_rows(getattr(self, name), _dev(a, self.device))
                continue
            dst = getattr(self, name)
            src = _dev(a, self.device)
            dst.view(-1).copy_(src.reshape(-1).view(dst.dtype))

    # -------------------------------------------------------------- paged rows
    def map_rows(self, b: int, n_rows: int, order=None) -> None:
        """Paged layers: give sequence b pages for compressed rows 0 ..
        n_rows - 1 (the blocks of positions 0 .. 256 ceil(n_rows / rpb) - 1)."""
        self.table.map_blocks(b, -(-n_rows // self.rpb), order)

    def release_sequence(self, b: int) -> None:
        """Paged layers: return sequence b's pages to the pool."""
        self.table.release(b)

    def _scatter_rows(self, pool: torch.Tensor, rows: torch.Tensor) -> None:
        nb = self.cap // self.rpb
        for b in range(self.batch):
            self.map_rows(b, self.cap)
            pages = self.table.dev[b].long()
            src = rows[b].reshape(nb, -1).view(torch.uint8)
            pool.view(pool.shape[0], -1).index_copy_(0, pages, src.reshape(nb, -1))

    def _gather_rows(self, pool: torch.Tensor, row_elems: int, dtype) -> torch.Tensor:
        nb = self.cap // self.rpb
        out = torch.zeros((self.batch, nb, pool[0].numel()), dtype=torch.uint8, device=self.device)
        for b in range(self.batch):
            pg = self.table.dev[b].long()
            ok = (pg >= 0) & (pg < pool.shape[0])
            out[b][ok] = pool.view(pool.shape[0], -1)[pg[ok]]
        return out.view(self.batch, self.cap, -1).view(dtype).view(self.batch, self.cap, row_elems)

    def comp_rows(self) -> torch.Tensor:
        """The K=V rows as [batch, comp_cap, row_bytes] (paged: gathered from
        the pages, zeros where a block has no page in the pool)."""
        if not self.paged:
            return self.comp
        return self._gather_rows(self.comp, self.rb, torch.uint8)

    def idx_rows(self) -> torch.Tensor:
        """The indexer rows in the contiguous layout's shape and type."""
        if not self.paged:
            return self.idx
        if self.idx_fmt == "fp4":
            return self._gather_rows(self.idx, self.irb, torch.uint8)
        dt = torch.float32 if self.idx_fmt == "f32" else torch.int16
        return self._gather_rows(self.idx, self.DI, dt)

    # -------------------------------------------------------------- steps
    def _stream(self):
        return torch.cuda.current_stream(self.device).cuda_stream

    def _check(self, rc: int, where: str):
        if rc != L.CKV_OK:
            raise L.CkvError(rc, where)

    def new_out(self, n: int) -> torch.Tensor:
        """An attention output buffer: [n, H, d] in act_fmt, or with
        CKV_FLAG_OUT_FP8 [n, H, d + 4 d/128] bytes of fp8 records."""
        if self.desc.flags & L.CKV_FLAG_OUT_FP8:
            return torch.empty((n, self.H, self.d + 4 * (self.d // 128)), dtype=torch.uint8, device=self.device)
        dt = torch.float32 if self.act_fmt == "f32" else torch.bfloat16
        return torch.empty((n, self.H, self.d), dtype=dt, device=self.device)

    def compress_decode(self, x, u, pos, B: Optional[int] = None) -> None:
        B = self.batch if B is None else B
        self._check(L.compress_append_decode(self.desc, self.weights, self.cache, x, u, pos, B, self.ws,
                                             self.ws_bytes, self._stream()), "compress_append_decode")

    def indexer_decode(self, qI, w, pos, topk, B: Optional[int] = None) -> None:
        B = self.batch if B is None else B
        self._check(L.indexer_topk_decode(self.desc, self.cache, qI, w, pos, B, topk, self.ws, self.ws_bytes,
                                          self._stream()), "indexer_topk_decode")

    def attn_decode(self, q, pos, topk, out, B: Optional[int] = None) -> None:
        B = self.batch if B is None else B
        self._check(L.sparse_swa_attn_decode(self.desc, self.cache, q, pos, topk, B, out, self.ws,
                                             self.ws_bytes, self._stream()), "sparse_swa_attn_decode")

    def decode(self, x, u, q, qI, w, pos, out=None, topk=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
        """One decode step for every sequence: compress_append -> indexer_topk
        (ratio 4) -> sparse_swa_attn.  All tensors on the device."""
        B = self.batch
        out = self.new_out(B) if out is None else out
        if self.ratio == 4 and topk is None:
            topk = torch.empty((B, self.k), dtype=torch.int32, device=self.device)
        self.compress_decode(x, u, pos)
        if self.ratio == 4:
            self.indexer_decode(qI, w, pos, topk)
        self.attn_decode(q, pos, topk if self.ratio == 4 else None, out)
        return out, (topk if self.ratio == 4 else None)

    def decode_step(self, x, u, q, qI, w, pos, out=None, topk=None,
                    B: Optional[int] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
        """The same step as ``decode`` through the single decode-step entry
        point (fused launches on eligible ratio-4 layers)."""
        B = self.batch if B is None else B
        out = self.new_out(B) if out is None else out
        if self.ratio == 4 and topk is None:
            topk = torch.empty((B, self.k), dtype=torch.int32, device=self.device)
        self._check(L.decode_step(self.desc, self.weights, self.cache, x, u, q, qI, w, pos, B,
                                  topk if self.ratio == 4 else None, out, self.ws, self.ws_bytes, self._stream()),
                    "decode_step")
        return out, (topk if self.ratio == 4 else None)

    def prefill(self, seq: int, pos0: int, x, u, q, qI=None, w=None, out=None,
                topk=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
        """Chunked prefill of tokens pos0 .. pos0+T-1 of sequence ``seq``."""
        T = u.shape[0]
        out = self.new_out(T) if out is None else out
        if self.ratio == 4 and topk is None:
            topk = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        st = self._stream()
        self._check(L.compress_append_prefill(self.desc, self.weights, self.cache, x, u, seq, pos0, T, self.ws,
                                              self.ws_bytes, st), "compress_append_prefill")
        if self.ratio == 4:
            self._check(L.indexer_topk_prefill(self.desc, self.cache, qI, w, seq, pos0, T, topk, self.ws,
                                               self.ws_bytes, st), "indexer_topk_prefill")
        self._check(L.sparse_swa_attn_prefill(self.desc, self.cache, q, seq, pos0, T,
                                              topk if self.ratio == 4 else None, out, self.ws, self.ws_bytes,
                                              st), "sparse_swa_attn_prefill")
        return out, (topk if self.ratio == 4 else None)

    def prefill_chunk(self, seq: int, pos0: int, x, u, q, qI=None, w=None, out=None, topk=None,
                      side_stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
        """The same chunk as :meth:`prefill` in one call (ckv_prefill_chunk); with
        ``side_stream`` (a torch stream) the indexer branch runs there beside
        the attention lane's compression and the raw staging."""
        T = u.shape[0]
        out = self.new_out(T) if out is None else out
        if self.ratio == 4 and topk is None:
            topk = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        side = None if side_stream is None else side_stream.cuda_stream
        self._check(L.prefill_chunk(self.desc, self.weights, self.cache, x, u, q, qI, w, seq, pos0, T,
                                    topk if self.ratio == 4 else None, out, self.ws, self.ws_bytes, self._stream(),
                                    side), "prefill_chunk")
        return out, (topk if self.ratio == 4 else None)
