"""MI355X-native fused chunked top-K KL distillation loss.

The compute lives in a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, declared in ``include/kd_topk_kl.h``); ``binding`` is a thin
ctypes layer with the same entry-point names.
"""
