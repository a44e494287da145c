"""CPU oracle for the fused mHC boundary: plain, slow, fp64.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it. It shares no code with the HIP library and
imports nothing from it.

Pages cited (by title and section):
  * boundary page  -- vllm.models.deepseek_v41.nvidia.specialized_decode.boundary.boundary
  * all_reduce page -- vllm.models.deepseek_v41.nvidia.specialized_decode.boundary.all_reduce
  * decode page    -- vllm.models.deepseek_v41.nvidia.specialized_decode.runtime.decode

The pages give the dataflow and the argument lists of the calls but print no
formula for the arithmetic; where a step is open, each function states the
reading it takes.

Parity status: every function here is pinned by a CPU test against a closed
form, an invariant, a brute-force loop or an independent library routine,
except the orientation of ``comb`` (which index is the output stream) and the
exact Sinkhorn convention (shift, order, placement of eps), which the pages do
not fix: for those two choices parity is unpinned by the pages, and only
self-consistency (plus the limit properties every convention shares) is tested.
"""

from . import codecs, mhc  # noqa: F401
from .codecs import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    e4m3_decode,
    e4m3_encode,
    e8m0_exponent,
    mxfp8_quantize,
)
from .mhc import (  # noqa: F401
    tp_reduce,
    moe_finalize_sum,
    mhc_post,
    collapse,
    rms_norm,
    boundary,
    finalize,
    residual_only,
    collapse_mean,
    first,
    collapse_norm,
    sinkhorn,
    pre_coeffs,
    decode_chain,
)
