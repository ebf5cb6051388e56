"""Prefix-shared attention forward for AMD MI355X (gfx950).

The computation lives in ``libpsattn.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/psattn.h``); ``psattn`` is a thin ctypes binding that
marshals PyTorch device tensors and the current HIP stream into that ABI.
"""
