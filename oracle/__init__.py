"""CPU oracle for one routed MoE layer served from a shared expert-slot cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import or run anything in this
package.  The HIP library never calls it and shares no code with it; the
only thing both sides share is the seeded input generators in ``harness/``.

What it computes, in plain float64 NumPy (slow on purpose, no blocking or
fusion beyond what the definitions state):

* ``route``   top-k routing with softmax over the kept logits
* ``qsplit``  the bandwidth split q* of cache misses between fills and host
* ``lru``     the shared LRU slot cache: dedup, hit/miss, victims, update,
              rewrite of routes to slots or to the host set
* ``numerics`` exact decoding of BF16 and OCP E4M3FN codes
* ``ffn``     the SwiGLU expert FFN and the gate-weighted layer output,
              split into GPU and host partial sums

Sources (the pages this reproduces; each function names its passage):
  [FT]  "FreeToken 完全拆解" (pinghaoyang.com.cn/aigc/posts/freetoken/)
  [FTK] "개인 장치에서 MoE 모델을 서빙하는 FreeToken" (aitrends.kr/articles/99620)
  [OSDI] "OSDI'26 | 双路 CPU + 两张 5090 ..." (marsggbo.github.io, 2026-07-23)

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against values the pages print, closed forms, library routines or brute
force (tests/test_oracle_pins.py), except the layer outputs on the five
synthetic workloads themselves, for which the pages print no values; those
are pinned only through the FFN's special cases and invariants.
"""
from . import numerics, route, qsplit, lru, ffn  # noqa: F401
