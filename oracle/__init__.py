"""CPU oracle for the MTP speculative-decoding step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it and shares no code with it.

The oracle is plain, slow and row-by-row: NumPy in float64, one row of one
sequence at a time, in the order the pages describe the method.  It exists so
that the device path has something obviously correct to be compared with.

Sources (web pages), cited by title and section:

* [HB14] "14. MTP: speculative decoding with the built-in draft head"
  (Transformer by Hand handbook, stage 2).  Sections: "The draft head" (the
  mtp.py listing and the prose after it), "Acceptance rate and speed-up".
* [DLM]  "The decoding loop and MTP" (agent-loop-visualizer docs).  Sections:
  "Why a hand-written decoding loop", "MTP speculative decoding" items 1-3.
* [YL]   "MTP (Multi-Token Prediction) 原理详解".  Sections 二 (module
  architecture), 三 (stages 0-4), 四 (worked example and counter-example),
  五 (design points).

Pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``; no function
here is left "parity unpinned".
"""
from .mtp import *  # noqa: F401,F403
