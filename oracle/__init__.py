"""fp64 CPU oracle of the GPTQ per-layer path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It is independent of the HIP library
(no shared code, headers, tables or helpers; neither imports the other).

Pinned functions (see ``tests/test_oracle_pins.py``): ``hessian``, ``damp``,
``hinv_cholesky_upper``, ``grid``, ``quantize_values``, ``quantize``,
``dequantize``, ``output_error``, ``pack_codes``, ``unpack_codes``,
``output_error_from_errors``, ``obq_quantize``, ``propagate``.  No function here is
"parity unpinned".
"""
from .gptq import (  # noqa: F401
    NotPositiveDefinite,
    ObqResult,
    QuantResult,
    damp,
    dequantize,
    grid,
    hessian,
    hinv_cholesky_upper,
    layer,
    obq_quantize,
    output_error,
    propagate,
    output_error_from_errors,
    pack_codes,
    prepare,
    quantize,
    quantize_values,
    unpack_codes,
)
