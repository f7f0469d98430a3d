"""fldce: fused linear diffusion cross-entropy (LM head) for MI355X (gfx950).

The compute path is the HIP library ``libfldce.so`` behind the C ABI declared
in ``include/fldce.h``; ``lm_head_linear_bf16_amd.fldce`` is its thin ctypes
binding.  Importing this package loads nothing; the binding loads the library
on first use and raises if it is missing.
"""
