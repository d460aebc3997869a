"""Host logic of the paged compressed caches (no GPU): rows per 256-position
block, free lists, block tables, the three page sizes of a c4a + c128a stack,
and the library's host checks of a paged cache description."""
import numpy as np
import pytest
import torch

from compressed_kv_sparse_amd import _lib as L
from compressed_kv_sparse_amd.paged import BLOCK_TOKENS, BlockTable, FreeList, PagePools, rows_per_block


def test_rows_per_block():
    assert BLOCK_TOKENS == 256
    assert rows_per_block(4) == 64 and rows_per_block(128) == 2
    with pytest.raises(ValueError):
        rows_per_block(0)


def test_free_list_order_and_errors():
    f = FreeList(4)
    assert [f.alloc() for _ in range(4)] == [0, 1, 2, 3]
    with pytest.raises(MemoryError):
        f.alloc()
    f.release([2, 0])
    assert f.n_free == 2 and f.alloc() == 0 and f.alloc() == 2
    with pytest.raises(ValueError):
        f.release([4])


def test_block_table_map_release_and_given_order():
    f = FreeList(10)
    t = BlockTable(f, batch=2, max_blocks=4, device="cpu")
    t.map_blocks(0, 2)
    assert t.host[0].tolist() == [0, 1, -1, -1] and f.n_free == 8
    t.map_blocks(0, 3)                       # only the new block takes a page
    assert t.host[0].tolist() == [0, 1, 2, -1]
    t.map_blocks(1, 2, order=[9, 5])         # scattered pages
    assert t.host[1].tolist() == [9, 5, -1, -1]
    assert torch.equal(t.dev, torch.from_numpy(t.host))
    with pytest.raises(ValueError):
        t.map_blocks(1, 3, order=[9])        # page 9 is taken
    with pytest.raises(ValueError):
        t.map_blocks(0, 5)                   # beyond comp_cap
    t.release(0)
    assert t.host[0].tolist() == [-1] * 4 and f.n_free == 10 - 2 + 0
    assert (t.dev[0] == -1).all()


def test_three_page_sizes_of_a_flash_stack():
    """fp8 K=V rows (640 B) and bf16 indexer rows (256 B): c4a K=V pages of 64
    rows, c4a indexer pages of 64 rows, c128a K=V pages of 2 rows."""
    rb = L.row_bytes(L.CKV_E4M3, 512)
    irb = L.idx_row_bytes(L.CKV_BF16, 128)
    p = PagePools(kv_row_bytes=rb, idx_row_bytes=irb, pages_c4a=8, pages_c128a=16, device="cpu")
    assert p.page_sizes() == {"c4a_kv": 64 * 640, "c4a_idx": 64 * 256, "c128a_kv": 2 * 640}
    assert p.n_pages(4) == 8 and p.n_pages(128) == 16
    # a c4a layer's K=V and indexer rows of one block share the page index:
    # one free list for both c4a pools
    assert set(p.free) == {4, 128}
    # one sequence of 131072 tokens: 512 blocks on every compressed layer
    assert 131072 // 256 == 512


def _desc(**kw):
    base = dict(ratio=4, hidden=4096, head_dim=512, n_rot=64, n_heads=64, swa=128, idx_heads=64, idx_dim=128,
                top_k=512, comp_cap=32768, batch=16, kv_fmt=L.CKV_E4M3, idx_fmt=L.CKV_BF16, act_fmt=L.CKV_BF16,
                w_fmt=L.CKV_BF16, flags=0, rope_base=160000.0, norm_eps=1e-6, softmax_scale=0.0)
    base.update(kw)
    return L.LayerDesc(**base)


FAKE = 1 << 40


def _cache(**kw):
    c = dict(raw=FAKE, comp=FAKE, idx=FAKE, st_kv=FAKE, st_sc=FAKE, ist_kv=FAKE, ist_sc=FAKE, raw_stage=FAKE,
             stage_rows=4096 + 127, status=None, block_table=FAKE, n_pages=100)
    c.update(kw)
    return L.LayerCache(**c)


@pytest.mark.skipif(__import__("os").path.exists("/dev/kfd"),
                    reason="fake device addresses are only passed where no GPU exists")
def test_paged_cache_host_checks():
    d = _desc()
    ws = L.workspace_bytes(d, L.CKV_MODE_DECODE, 16)
    call = lambda c, dd=d: L.indexer_topk_decode(dd, c, FAKE, FAKE, FAKE, 16, FAKE, FAKE, 1 << 20)
    assert call(_cache(block_table=FAKE + 2)) == L.CKV_E_INVAL        # misaligned table
    assert call(_cache(n_pages=0)) == L.CKV_E_INVAL                   # empty pool
    # comp_cap must hold whole blocks: 64 rows (c4a), 2 rows (c128a)
    assert call(_cache(), _desc(comp_cap=32768 - 32)) == L.CKV_E_UNSUPPORTED
    d128 = _desc(ratio=128, comp_cap=1025, kv_fmt=L.CKV_BF16)
    assert L.sparse_swa_attn_decode(d128, _cache(), FAKE, FAKE, None, 16, FAKE, FAKE, 1 << 30) == \
        L.CKV_E_UNSUPPORTED
    # a window-only layer has no compressed rows: the table is ignored
    d0 = _desc(ratio=0, comp_cap=0)
    assert L.sparse_swa_attn_decode(d0, _cache(n_pages=0), FAKE, FAKE, None, 16, FAKE, FAKE, 1) == \
        L.CKV_E_WORKSPACE
    assert ws > 0
