"""MI355X (gfx950) implementation of Lynx's hierarchical split-stream KV
quantizer: bf16 KV page blocks -> 4-bit anchor + 4-bit residual streams and
per-page metadata, and the anchor-only / anchor+residual reconstructions.

The compute runs in hand-written HIP kernels behind the C ABI of
``include/lynx.h`` (``liblynx.so``); ``progressive_kv_transfer_amd.lynx`` is
the thin Python binding over it.  Importing this package loads nothing; the
first call into ``lynx`` loads the library and fails loudly if it is missing.
"""
