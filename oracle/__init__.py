"""CPU oracle for the Delta-CoMe mixed-precision delta apply.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The
library under ``tenant_rank_serving_amd/`` never imports, links or calls it,
and this package shares no code with it: it is a second, independent,
deliberately plain implementation written from the pages, in numpy fp64.

Pages cited (by title, then section):
  [P1] "Delta-CoMe - 清华联合OpenBMB等高校开源的新型增量压缩算法" (paooo.com news
       article): sections "Delta-CoMe的技术原理" (technical principles) and
       "Delta-CoMe的应用场景" (application scenarios).
  [P2] "Delta-CoMe: Training-Free Delta-Compression with Mixed-Precision for
       Large Language Models" (atlas.scime.ai summary): "Problem",
       "Approach", "Key results", "Experimental setup" (Builds on: GPTQ).
  [P4] "Enhancing Delta Compression in LLMs via SVD-based Quantization Error
       Minimization" (gist.science explainer of the follow-up PrinMix): §2.1
       (W = U Sigma V, row-wise quantization of V; eq. 5, the error of a
       row), §2.2 (bit allocation as a 0/1 integer program), §2.4 (pipeline).

What the pages fix and what they leave open is listed per function.  Where
they are silent the reading taken is marked [R]; every [R] is also listed in
the design notes of the repository.

Modules:
  quant   SVD into singular pairs, rank groups, RTN quantizer, dequantizer
  layout  the packed byte format (pack / unpack)
  apply   y = W x + U diag(sigma) V x in fp64, brute-force loop, routing
  alloc   bit allocation: eq. 5 errors, exact knapsack program, brute force

Every function here is pinned by a test in tests/test_oracle_*.py against
something other than itself (closed forms, hand-derived values, brute force,
special cases); none is "parity unpinned".
"""
from . import quant, layout, apply  # noqa: F401
