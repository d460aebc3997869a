"""Seeded device-side draws for timing runs of many layers.

The host generator (``gen.py``) is the one the parity tests use; it draws a
128k-context c4a layer in seconds, which is too slow for a 43-layer stack.
The functions here fill a layer's cache tensors directly on the device with
the same laws (see ``gen.py``):

* bf16 values are the high 16 bits of float32 normal draws;
* fp8 E4M3 codes take sign and octave from a normal draw (exponent field
  floor(log2|g|) + 13, clipped to 1..15) and 3 uniform mantissa bits, never
  the NaN pattern;
* the per-row fp32 scale is U(0.75/64, 1.25/64);
* window state is N(0, 1) fp32; indexer head weights are U(0, 1).

The values differ from the host draws (another generator), so these inputs
serve timing only.  Nothing here projects, pools, normalises, rotates,
scores, selects or attends.
"""
from __future__ import annotations

import zlib

import torch

from .gen import FP4_SCALE_BYTES, e4m3_row_offsets


def _gen(seed: int, name: str, layer: int) -> torch.Generator:
    g = torch.Generator(device="cuda")
    g.manual_seed((seed * 1_000_003 + (zlib.crc32(name.encode()) & 0x7FFFFFFF) * 131 + layer) & 0x7FFFFFFFFFFF)
    return g


def bf16_draw(shape, g: torch.Generator, std: float = 1.0) -> torch.Tensor:
    """int16 tensor of bf16 bit patterns (high half of a float32 normal draw)."""
    a = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    if std != 1.0:
        a.mul_(std)
    return (a.view(torch.int32) >> 16).to(torch.int16)


def e4m3_codes(shape, g: torch.Generator) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    sign = (x < 0).to(torch.int32)
    e = torch.floor(torch.log2(x.abs().clamp_min(1e-30))).to(torch.int32).add_(13).clamp_(1, 15)
    m = torch.randint(0, 8, shape, generator=g, device="cuda", dtype=torch.int32)
    m = torch.where((e == 15) & (m == 7), torch.full_like(m, 6), m)
    return ((sign << 7) | (e << 3) | m).to(torch.uint8)


def fill_rows(dst: torch.Tensor, fmt: str, d: int, n_rot: int, g: torch.Generator) -> None:
    """Fill uint8 row records dst[..., row_bytes] with drawn rows of format ``fmt``."""
    shape = tuple(dst.shape[:-1])
    if fmt == "bf16":
        dst.copy_(bf16_draw(shape + (d,), g).view(torch.uint8).reshape(dst.shape))
        return
    if fmt == "f32":
        dst.copy_(torch.randn(shape + (d,), generator=g, device="cuda").view(torch.uint8).reshape(dst.shape))
        return
    dn = d - n_rot
    toff, soff = e4m3_row_offsets(d, n_rot)
    dst.zero_()
    dst[..., :dn] = e4m3_codes(shape + (dn,), g)
    dst[..., toff:toff + 2 * n_rot] = bf16_draw(shape + (n_rot,), g).view(torch.uint8).reshape(shape + (2 * n_rot,))
    sc = torch.empty(shape, device="cuda", dtype=torch.float32).uniform_(0.75 / 64, 1.25 / 64, generator=g)
    dst[..., soff:soff + 4] = sc.view(torch.uint8).reshape(shape + (4,))


def fill_fp4_records(dst: torch.Tensor, dim: int, g) -> None:
    """fp4 indexer records as gen.draw_fp4_records lays them out: uniform
    4-bit codes, block-scale bytes uniform in FP4_SCALE_BYTES."""
    lo, hi = FP4_SCALE_BYTES
    dst[..., :dim // 2].copy_(torch.randint(0, 256, tuple(dst.shape[:-1]) + (dim // 2,), generator=g,
                                            device="cuda", dtype=torch.int32).to(torch.uint8))
    dst[..., dim // 2:].copy_(torch.randint(lo, hi + 1, tuple(dst.shape[:-1]) + (dim // 32,), generator=g,
                                            device="cuda", dtype=torch.int32).to(torch.uint8))


def fill_layer_cache(dl, cfg) -> None:
    """Fill every cache tensor of a DeviceLayer as at a warm context (all rows
    drawn); every sequence has stored n_ctx - 1 tokens, so the step's token
    sits at position n_ctx - 1."""
    s, L = cfg.seed, cfg.layer
    dl.n_tokens.fill_(cfg.n_ctx - 1)
    fill_rows(dl.raw, cfg.kv_fmt, cfg.head_dim, cfg.n_rot, _gen(s, "raw", L))
    paged = getattr(dl, "paged", False)   # rows drawn in the contiguous shape, then scattered into pages
    if dl.comp is not None:
        comp = torch.empty((dl.batch, dl.cap, dl.rb), dtype=torch.uint8, device="cuda") if paged else dl.comp
        fill_rows(comp, cfg.kv_fmt, cfg.head_dim, cfg.n_rot, _gen(s, "comp", L))
        if paged:
            dl.load_cache(comp=comp)
        dl.st_kv.normal_(generator=_gen(s, "st_kv", L))
        dl.st_sc.normal_(generator=_gen(s, "st_sc", L))
    if dl.idx is not None:
        idx = torch.empty_like(dl.idx_rows()) if paged else dl.idx
        if cfg.idx_fmt == "bf16":
            idx.copy_(bf16_draw(tuple(idx.shape), _gen(s, "idx", L)))
        elif cfg.idx_fmt == "fp4":
            fill_fp4_records(idx, cfg.idx_dim, _gen(s, "idx", L))
        else:
            idx.normal_(generator=_gen(s, "idx", L))
        if paged:
            dl.load_cache(idx=idx)
        dl.ist_kv.normal_(generator=_gen(s, "ist_kv", L))
        dl.ist_sc.normal_(generator=_gen(s, "ist_sc", L))


def draw_weights(cfg) -> dict:
    """Per-layer compressor weights as device tensors (the laws of make_layer_weights)."""
    if cfg.ratio == 0:
        return {}
    s, L = cfg.seed, cfg.layer
    d, D, W = cfg.head_dim, cfg.hidden, cfg.window
    w_std = cfg.w_std if cfg.w_std is not None else D ** -0.5
    ape_std = cfg.ape_std if cfg.ape_std is not None else d ** -0.5

    def gamma(n, name):
        gm = torch.ones(n, device="cuda")
        if cfg.gamma_std:
            gm.add_(torch.randn(n, generator=_gen(s, name, L), device="cuda") * cfg.gamma_std)
        return gm

    out = dict(wkv=bf16_draw((d, D), _gen(s, "wkv", L), w_std), wgate=bf16_draw((d, D), _gen(s, "wgate", L), w_std),
               ape=torch.randn((W, d), generator=_gen(s, "ape", L), device="cuda") * ape_std,
               gamma=gamma(d, "gamma"))
    if cfg.ratio == 4:
        DI = cfg.idx_dim
        out.update(idx_wkv=bf16_draw((DI, D), _gen(s, "idx_wkv", L), w_std),
                   idx_wgate=bf16_draw((DI, D), _gen(s, "idx_wgate", L), w_std),
                   idx_ape=torch.randn((8, DI), generator=_gen(s, "idx_ape", L), device="cuda") * DI ** -0.5,
                   idx_gamma=gamma(DI, "idx_gamma"))
    return out


def draw_step_inputs(cfg) -> dict:
    """x, u, q (bf16 bits), q^I, w and positions for one decode step of every sequence."""
    s, L, B = cfg.seed, cfg.layer, cfg.batch
    out = dict(x=bf16_draw((B, cfg.hidden), _gen(s, "x", L)), u=bf16_draw((B, cfg.head_dim), _gen(s, "u", L)),
               q=bf16_draw((B, cfg.n_heads, cfg.head_dim), _gen(s, "q", L)),
               pos=torch.full((B,), cfg.n_ctx - 1, dtype=torch.int32, device="cuda"), qI=None, w=None)
    if cfg.ratio == 4:
        out["qI"] = bf16_draw((B, cfg.idx_heads, cfg.idx_dim), _gen(s, "qI", L))
        out["w"] = torch.rand((B, cfg.idx_heads), generator=_gen(s, "w", L), device="cuda")
    return out
