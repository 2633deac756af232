"""CPU oracle for FlashHead inference — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct float64 implementation of what the FlashHead
retrieval head computes, written stage by stage from the method's description
(FlashHead explainer, framerc.cn, §1.2 and §2.2.2; arXiv 2603.14591 abstract).
It shares no code with the HIP path and imports nothing from it.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never routes through it: the HIP
library fails loudly when it is missing instead of falling back here.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (closed forms, brute force, library routines, rocRAND's Philox);
see ``tests/test_oracle_*.py``.
"""

from .flashhead_oracle import (  # noqa: F401
    MODE_PROBE_SAMPLE,
    MODE_PROBE_SHARED,
    MODE_TOKEN_SAMPLE,
    OracleHead,
    dense,
    dequantize_g32,
    dequantize_int4,
    dequantize_int8,
    e4m3_decode,
    e4m3_encode,
    finish,
    forward,
    gather,
    pack_int4,
    probs_fp8,
    quantize_int4_g32,
    quantize_int8_g32,
    score,
    select,
    select_adaptive,
    select_shared,
    unpack_int4,
    validate_c2t,
)
from .philox import gumbel, philox4x32_10, uniform_from_word  # noqa: F401
from . import cluster_oracle  # noqa: F401,E402  (balanced k-means, the offline step)
from . import spec_oracle  # noqa: F401,E402  (speculative sampling: FlashHead draft, dense target)
