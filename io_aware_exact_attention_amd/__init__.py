"""Exact tiled softmax attention for MI355X (gfx950): HIP kernels behind a C ABI."""
