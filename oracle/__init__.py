"""CPU oracle for GPTQ layer quantization (float64 numpy).

TEST INFRASTRUCTURE: only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library and does not import it.
"""
from .gptq_ref import (  # noqa: F401
    GPTQResult, NotPositiveDefinite, act_order, damp, gptq, group_params, hessian,
    hinv_factor, n_groups, objective, pack_int4, quantize, rtn, unpack_int4,
)
