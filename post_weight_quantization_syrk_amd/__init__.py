"""GPTQ per-layer quantization hot path for AMD MI355X (gfx950).

The compute path lives in the HIP shared library ``libgptq_mi355x.so`` (sources
under ``csrc/``, C ABI in ``include/gptq.h``); ``gptq`` is its thin ctypes
binding.  ``synth`` generates the seeded synthetic inputs.
"""
__all__ = ["gptq", "synth"]
