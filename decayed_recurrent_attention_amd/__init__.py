"""Lightning (decayed recurrent) attention forward pass for AMD MI355X (gfx950).

The compute path is the HIP library ``liblattn.so`` behind the C ABI declared in
``include/lattn.h``; ``decayed_recurrent_attention_amd.lattn`` is its Python
binding.  Importing this package loads nothing; the library is loaded on first
use and a missing library is an error, never a silent fallback.
"""
__all__ = ["lattn", "inputs"]
