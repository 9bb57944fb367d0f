"""Plain, slow, fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only the test suite, the graft smoke entry and the benchmark's
``cpu_baseline`` leg use it.  It shares no code with the HIP library.

The oracle evaluates the definition of attention directly (no tiling, no
online softmax): every score row is materialised in full, an explicit boolean
mask selects the visible keys, and a max-subtracted softmax gives the output
and the log-sum-exp.

Sources (web pages on IO-aware exact attention):
  * "算子与编译器：FlashAttention 与长上下文" (charles2530 blog), §1 -- the
    attention formula softmax(Q Kᵀ/√d) V.
  * xxqk.cn article on FlashAttention for sliding-window prefill, §2 (formula),
    §4 (the bidirectional band and its causal variant), §5.2 (masked scores
    are -inf before the softmax).
  * "FlashAttention 深度解析：大模型长序列的算力解放" (ruiowl.com), §三 -- the
    tiled method is exactly equal to the standard computation, so the plain
    definition is the thing to compare against.

Every function here is pinned by the CPU test suite against brute force,
a library routine, closed forms and invariants; see tests/test_oracle_*.py.
"""

from .attention import (  # noqa: F401
    visible_mask,
    attention_rows,
    attention_fwd,
    decode_fwd,
    gather_paged_kv,
)
from .attention_bwd import (  # noqa: F401
    attention_bwd,
    attention_bwd_keys,
    attention_bwd_rows,
    probabilities,
)
from .varlen import attention_paged_prefill, attention_varlen  # noqa: F401
from .blocksparse import attention_block_sparse, attention_masked  # noqa: F401
from .fp8 import decode_fwd_fp8, e4m3_to_float  # noqa: F401
