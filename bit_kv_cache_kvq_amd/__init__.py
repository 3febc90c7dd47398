"""bit_kv_cache_kvq_amd -- low-bit quantized KV-cache decode attention for MI355X (gfx950).

The compute path is the C-ABI library ``libkvq.so`` (hand-written HIP kernels, see
``csrc/`` and ``include/kvq.h``).  ``binding`` marshals arguments to it with ctypes;
PyTorch is used only for device memory and streams.  ``synth`` draws the seeded
synthetic workloads.
"""
__all__ = ["binding", "synth"]
