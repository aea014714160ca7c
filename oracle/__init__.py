"""CPU oracle for the grouped 4-bit mixture-of-experts matmul.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct reference that the HIP path is checked against.  Only the test
suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it; the product path (``bit_grouped_moe_amd``)
never does, and it shares no code, table or helper with the kernels.

Everything here is NumPy on the host, in float64 wherever the method does
floating-point arithmetic and the pages do not fix another precision.
Each function cites the web page (by title) and the section it follows:

* "grouped-nf4-gemm 0.43.0" (PyPI project page) -- sections "Which entry
  point?" and "Try the packers and byte checks on CPU";
* "Receipts-driven engineering" -- the opening summary of what the kernel
  computes;
* "How do I run MoE expert inference natively on MXFP4 (e2m1 + e8m0)
  weights ..." -- its summary;
* "flashrt/grouped-moe-gemv" -- section "Functions" (routing tensor and
  output layout conventions).

``fp8`` holds the e4m3 element format and the two-term activation split
that the block-scaled fp4 matmul path uses (a reading: the pages keep the
activations in bf16; see that module's docstring).

Where the pages are silent the reading taken is stated in the docstring of
the function concerned.

Parity status: every public function is pinned by CPU tests against
values or identities the pages and mathematics fix (printed shapes and
round-trip errors, closed forms, brute force on tiny inputs, adjoint
identities, a library routine for bf16 rounding).  No function here is
"parity unpinned".
"""

from .bf16 import f32_to_bf16_rne, bf16_to_f32  # noqa: F401
from .nf4 import NF4_CODEBOOK, nf4_pack, nf4_decode  # noqa: F401
from .mxfp4 import E2M1_VALUES, e2m1_value, mxfp4_pack, mxfp4_decode  # noqa: F401
from .fp8 import (E4M3_VALUES, e4m3_value, e4m3_rne, block_scale_exponent,  # noqa: F401
                  act_split_e4m3, act_split_value)
from .route import route_sort  # noqa: F401
from .grouped import (  # noqa: F401
    grouped_gemm,
    grouped_dgrad,
    brute_force_gemm,
    brute_force_dgrad,
    compare_slices,
    REL_L2_TOL,
)
from .moe import (silu, swiglu, gate_up_swiglu, combine, down_combine, OSS_ALPHA,  # noqa: F401
                  OSS_LIMIT, swiglu_oss, gate_up_swiglu_oss)
