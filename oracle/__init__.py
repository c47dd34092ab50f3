"""CPU oracle for the fused SRFT/SRHT int4 KV-cache quantizer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
executes this package: only the test suite (``tests/``), the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
use it.  It shares no code, table or constant generator with the HIP library
under ``kv_cache_int4_amd/``; the two meet only in the seeded input
generators, which hold none of the method's arithmetic.

The oracle is plain, slow and written to be checked by eye against the
sources it cites: numpy in float64 for the rotations and the attention
softmax, numpy's IEEE float32/float16 arithmetic where a floating-point value
decides an integer (a group scale or a code), and pure-Python loops for the
brute-force cross-checks.  See ``oracle/kvq_oracle.py``.

Source pages (cited by title and section):
  * "When Quantization Is Free: An int4 KV Cache That Outruns fp16 on Apple
    Silicon" (M. A. Bergach, arXiv 2605.05699) -- its abstract, as shown on
    the paperdance.org and mlsanity.com pages;
  * the gist.science explainer of the same paper, "Technische
    Zusammenfassung", sections "Methodik" 1-3 and "Speichereffizienz";
  * "Quantization Dominates Rank Reduction for KV-Cache Compression"
    (arXiv 2604.11501), abstract.
"""

from .kvq_oracle import *  # noqa: F401,F403
from .kvq_oracle import __all__  # noqa: F401
