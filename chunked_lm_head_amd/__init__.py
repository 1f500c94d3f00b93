"""Chunked fused linear cross-entropy / selective log-softmax for MI355X (gfx950).

The compute lives in a HIP shared library behind a C ABI (``include/flce.h``);
``chunked_lm_head_amd.flce`` is the thin ctypes binding.  Importing this package
does not load the library: ``from chunked_lm_head_amd import flce`` does.
"""
__all__ = ["flce", "synth"]
