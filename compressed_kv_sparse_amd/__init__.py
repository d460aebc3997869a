"""MI355X-native compressed-KV sparse attention (DeepSeek-V4 style c4a / c128a).

The compute lives in libckv.so (hand-written HIP for gfx950) behind the C ABI
of include/ckv.h; this package is its Python binding.  Importing it loads the
library and raises ImportError when it has not been built.
"""
from . import _lib  # noqa: F401  (loads libckv.so or raises)
from ._lib import (  # noqa: F401
    CkvError, LayerCache, LayerDesc, LayerWeights, FMT, compress_append_decode, compress_append_prefill,
    indexer_topk_decode, indexer_topk_prefill, row_bytes, sparse_swa_attn_decode, sparse_swa_attn_prefill,
    strerror, validate, workspace_bytes,
)
from .hc import HCMixer  # noqa: F401
from .layer import DeviceLayer  # noqa: F401
from .paged import BlockTable, FreeList, PagePools, rows_per_block  # noqa: F401
