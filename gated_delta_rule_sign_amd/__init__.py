"""Complex KDA (CKDA) recurrence on AMD Instinct MI355X (gfx950).

The compute path is ``libckda.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/ckda.h``); ``gated_delta_rule_sign_amd.ckda`` is the thin
ctypes binding over it.  Importing this package loads nothing; the binding
loads the library on first use and raises if it is missing.
"""
__all__ = ["inputs", "ckda"]
