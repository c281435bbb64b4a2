"""Batch-1 decoder-layer engine for AMD MI355X (gfx950).

``lib`` binds the C ABI of libdec (HIP kernels); ``engine`` holds a decode
stack's device state and per-token graph. Build the library with
``python -m transformer_layer_amd.build``.
"""
