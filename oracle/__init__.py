"""CPU oracle for Attn-QAT attention (plain, slow, float64 numpy).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything in this package. It shares no code with the HIP library
(``quantization_aware_attention_amd``) and never imports it; the two meet only
through the seeded inputs of the ``synthetic`` package.

Modules:

* ``nvfp4``        NVFP4 fake quantization (E4M3 scale per 16 elements, E2M1
                   values, no global scale).
* ``attention``    dense forward (O, LSE) and straight-through backward.
* ``block_sparse`` VSA-style block selection and block-sparse fine attention.

Parity pins (tests marked ``not gpu``) tie every function to something other
than itself: exhaustive exact-rational rounding checks, the E4M3 cast of a
library, closed forms of uniform attention, textbook attention and autograd
with quantization off, central finite differences of the straight-through
surrogate, and brute-force selection. See ``tests/test_oracle_*.py``.
Parity unpinned: agreement with FastVideo's own kernels (the pages give neither
code nor numeric outputs for them).
"""
from . import attention, block_sparse, nvfp4  # noqa: F401
