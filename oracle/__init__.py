"""CPU oracle for the W4A16 routed-expert layer — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package never
imports the product path. The arithmetic lives in ``oracle.c`` (plain C, fp64
forward, fp32 quantiser decisions); this module only marshals numpy arrays.
Everything exported here computes something the pages define; the library's
own tiled weight layout (a load order of the GPU kernels, no page defines it)
is described in the tests' helper ``tests/tiled_layout.py``, not here.
Functions with no independent pin are marked "parity unpinned" in oracle.c's
header and in the design doc (the gate/up row order and the choice of GELU(tanh)
as the activation).
"""
from .api import (  # noqa: F401
    build,
    load,
    f32_to_f16,
    f16_to_f32,
    quantize_rtn,
    dequant,
    align,
    router,
    w4a16_linear,
    moe_forward,
    gelu_tanh,
    threads,
    set_threads,
    philox4x32_10,
    gumbel_uniform,
    gumbel_score,
    sample,
)
