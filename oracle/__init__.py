"""CPU oracle for the block-draft round.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
imports, calls or links anything here, and nothing here imports the product.

The oracle is plain, slow and written to be checked by eye against the pages:
float64 arithmetic over the (bf16- or fp32-valued) inputs, NumPy library
primitives (matmul, exp, sort, cumsum, searchsorted) as single steps, and no
blocking, fusion or reordering beyond what each definition states.

Sources (cited by page title and section):
  * "The Next Generation of Speculative Decoding: DFlash and Spec V2"
    (lmsys.org blog digest; called *DFlash/Spec V2 blog* below) -- the KV
    injection formula (summary, A1, A2) and immediate materialization with a
    layer-batched projection plus fused Norm+RoPE post-processing (A7).
  * "Didi EAGLE-3 training/inference practice" (called *Didi EAGLE-3 article*),
    section 5.3 -- merging partial attention results with log-sum-exp so the
    result equals one global softmax.
  * DeepSeek DSpark tutorial (called *DSpark tutorial*), "speculative decoding
    basics" -- prefix acceptance, resampling at the first divergence, one extra
    token per round, losslessness; "confidence-scheduled verification" -- the
    per-position acceptance probability 1 - 1/2 |p_d - p_t|_1.
  * "Tencent open-sources DSpine" (called *DSpine article*) -- block of 16 = 1
    anchor + 15 drafted positions and an 8192-token sliding window ("what these
    weights are"); bidirectional in-block attention of DFlash ("principle");
    temperature 1.0 / top-p 0.95 / top-k 20 ("speed-up"); batched-verification
    rounding flips near-tied tokens ("tuning and memory").

Every function has at least one pin in ``tests/test_oracle_*.py`` (closed
forms, invariants, brute force, library routines, hand-derived fixtures in
``tests/golden/``); none is "parity unpinned".
"""
from . import bf16, inject, attention, verify  # noqa: F401

__all__ = ["bf16", "inject", "attention", "verify"]
