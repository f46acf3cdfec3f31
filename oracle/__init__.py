"""CPU oracle for the emulated-peer AllReduce — TEST INFRASTRUCTURE ONLY.

This package is the checker, not the product.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call, link or execute anything in it.  It shares no code with the HIP
path (``allreduce_emulated_peer_amd``) and imports nothing from it; the two
meet only through the seeded input generator module, which holds none of the
method's arithmetic.

What it computes (plain definition, no blocking or reordering beyond it):

* The pages name AllReduce as the collective MSCCL++ accelerates in
  tensor-parallel LLM inference (MSCCL++ project summary, "Highlighted
  Details"), inside a collective library with the usual collective
  interface (MSCCL++ ASPLOS'26 abstract).  A standard AllReduce with the sum
  operator leaves every rank holding the element-wise sum of all ranks'
  buffers.
* The pages fix no accumulation type, order or rounding.  Reading taken:
  each element is accumulated in IEEE binary32, starting from rank 0's value
  converted exactly to binary32 and adding ranks 1..R-1 in that order, each
  add rounded to nearest-even; the binary32 total is then rounded once to the
  element type (round-to-nearest-even, subnormals kept, NaN/Inf propagated).
  The result is replicated to all R outputs.

The same module also defines the two halves of the collective as standard
collectives of their own: ReduceScatter (rank r receives block r of the sum,
same accumulation rule) and AllGather (every rank receives all ranks' blocks
in rank order, bit for bit).

Modules:
  allreduce.py      NumPy implementation (the authority).
  allreduce_cpu.c   The same definition in plain C over host threads, used
                    for full-size checks and the timed CPU baseline; it is
                    checked bit-for-bit against allreduce.py.
  build.py          Compiles allreduce_cpu.c with gcc (no fast-math, no FP
                    contraction).

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts
that do not come from the oracle itself (closed forms, exact rational sums,
a scalar brute force, library rounding routines, invariants).
"""
