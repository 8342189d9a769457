"""MI355X-native paged KV cache: slot-mapping scatter, block-table gather and
fused paged decode attention, as hand-written HIP kernels for gfx950 behind a
small C ABI (include/pagedkv.h).  This package is the thin Python binding;
PyTorch only supplies device memory and streams."""
