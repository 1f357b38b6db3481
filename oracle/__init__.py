"""fp64 CPU oracle for streaming block-causal chunk attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library never
calls it and shares no code with it; both sides only share the seeded input
generators in ``synth``.

What it computes, and where the pages define it (pages cited by title and
section; the pages carry no formula, so each step below is the plainest
reading of the prose):

* Bounded cache -- "Vidu S2 vs PixVerse R2" blog (orkas.ai), section "Choice 3:
  bounded memory" (选择三：有上限的记忆): the first blocks stay as permanent
  sinks, a sliding window keeps the most recent blocks, older ones are dropped,
  so the cost of a new block does not grow with the stream.  ``cache.py``.
* Block causality -- same blog, section "What real-time changes" (「实时」改变了
  什么): blocks are generated in time order and a block sees only earlier
  content; the Vidu S2 paper read (yingwang.github.io), section 2.2 (数字人模型
  的训练): a segment sees the reference, its own condition and the history.
  Read as: bidirectional inside the current block, causal across blocks.
* 3D RoPE -- paper read, abbreviation table (RoPE entry): rotary positions over
  space and time.  RoPE relocation / relative-time RoPE -- blog "Choice 3":
  positions stay inside the range seen in training however long the session.
  ``rope.py``.
* TwinCache -- blog "Choice 3": every history block is cached noisy and clean;
  intermediate denoising steps read the noisy copy, the final step the clean
  one.  ``stream.py``.
* Block-sparse attention -- blog "Choice 4: where speed comes from" (选择四):
  learned block-sparse attention above 90% sparsity; here a top-k of
  mean-pooled tile scores on 128x128 tiles with forced tiles.  ``tilemask.py``.
* Attention itself -- scaled dot-product softmax attention, the textbook
  definition (the pages name attention but print no formula).  ``attention.py``.
* Variable-length blocks -- blog, section "Choice 5: how people control it":
  block length follows the control signal up to a cap.  ``rope.py``,
  ``stream.py``.
* Frame-aligned editing attention -- paper read, section 2.6 (the editing
  model); BloomBook Vidu S2 tutorial, section "S2-Editing".  ``stream.py``,
  ``bruteforce.py``.
* RMSNorm of q and k fused with the append -- paper read, section 2.4 (kernel
  fusion).  ``qknorm.py``.
* fp8 attention -- paper read, section 2.4 (quantised attention chosen per
  layer); an own E4M3 scheme with power-of-two group scales.  ``fp8.py``.

Pins (tests/test_oracle_*.py) tie each function to something other than itself:
closed forms, library routines, brute force over the whole stream with an
explicit block mask, and hand-computed worked examples under tests/golden/.
"""
from . import attention, bruteforce, cache, fp8, qknorm, rope, stream, tilemask  # noqa: F401
