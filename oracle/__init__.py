"""CPU oracle for exact attention and the softmax algorithms it is built on.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library under ``io_aware_softmax_06_amd/``; the only thing both sides
consume is the seeded inputs from ``workloads/``.

Everything here is plain NumPy in float64 (pure-Python loops where the method
itself is a sequential recurrence, used on small vectors only).  It is meant to
be slow and checkable by eye against the pages it follows:

  [P1] "FlashAttention", AllenY's blog (alleny.xyz/post/flashattention):
       sections "(Safe) Softmax", "从3-pass到2-pass" (from 3-pass to 2-pass),
       "FlashAttention" (one-pass fused form and the tiled loop).
  [P2] the wmrh.cn article on FlashAttention (wmrh.cn/news/298785):
       sections 2.1 "Online Softmax" (worked example on the vector [2, 1, 3])
       and 2.2 "把 Online Softmax 嵌入注意力" (online softmax inside attention).
  [P3] "理解 Flash Attention：在 Triton 中从头编写算法" (cnblogs, a translation
       of alexdremov.me): sections "什么是注意力？" (the attention formula),
       "瓦片注意力计算" (tiled attention; the rule for the softmax of a
       concatenation [x1, x2]; shift invariance), "算法概述" (one Q block per job).

Modules:
  softmax    -- naive, safe 3-pass, 2-pass online, element-streaming and
                block-merge softmax; the per-block statistics merge rule.
  exact_attention -- the definition O = softmax(scale * Q K^T [+ causal mask]) V with
                its natural-log logsumexp L (materialised S, fp64); a per-row
                form for sampled checks at full size; the tiled one-pass online
                algorithm in the pages' order (used only to show that it
                reaches the definition); the partial result over a key range
                and the merge of partials; the definition under a block mask
                (block-sparse attention, [P3] introduction).
  backward   -- the gradients dQ, dK, dV of <dO, O> by the chain rule through
                the row softmax, with S and P materialised ([P3] core idea:
                recompute the score matrix in the backward pass).

Pins: every function here is checked in ``tests/test_oracle.py`` against
something other than itself (closed forms, brute force with ``math.fsum``,
library special cases, invariants and the worked example of [P2] 2.1).  No
function is "parity unpinned".
"""

from .softmax import (  # noqa: F401
    softmax_naive,
    softmax_3pass,
    online_normaliser_states,
    softmax_2pass_online,
    softmax_stats,
    merge_stats,
    softmax_blocked,
)
from .exact_attention import (  # noqa: F401
    attention,
    attention_rows,
    attention_online_tiled,
    attention_partial,
    merge_partials,
    attention_block_sparse,
    attention_block_sparse_rows,
    expand_block_mask,
)
from .backward import attention_backward  # noqa: F401
