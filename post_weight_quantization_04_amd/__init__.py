"""GPTQ per-layer quantization path for AMD Instinct MI355X (gfx950).

The arithmetic lives in the HIP library ``libgptq_mi355x.so`` (C ABI in
``include/gptq.h``); ``_lib`` binds it with ctypes and ``layer`` drives the
three entry points with torch-allocated device buffers.  Build the library
with ``python -m post_weight_quantization_04_amd.build``.
"""
from ._lib import (  # noqa: F401
    GptqError,
    hessian_accumulate,
    kernel_names,
    load,
    prepare_hinv,
    prepare_hinv_workspace,
    quantize_layer,
    quantize_layer_workspace,
    status_string,
    timing_enable,
    timing_read,
)
