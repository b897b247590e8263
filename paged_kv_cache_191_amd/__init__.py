"""Attention over a block-paged KV cache (PagedAttention) and its
contiguous-KV counterpart (the vAttention layout), as hand-written HIP
kernels for MI355X (gfx950) behind a C ABI (``include/kvpaged.h``)."""
