"""fp64 CPU oracle for one ring rank's share of causal blockwise attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (``ring_attention_ra_amd``) never imports it, and this
package imports nothing from the product path: the two share no code.

What it computes is the plain definition of softmax attention over the
materialised global sequence, restricted to the query rows that one rank of a
ring holds. Every function cites the passage of the source pages it follows.
Pages are cited by host and section:

* discosf.com  -- practitioner article on context parallelism and Ring
  Attention (article heading "百万Token上下文训练的挑战与突破").
* digipub.cc   -- "大模型如何訓練百萬 Token 上下文：上下文并行與 Ring Attention".
* intelliparadigm.com -- long-context survey (positional encodings, including
  RoPE in ``rope_fp64``, and FlashAttention).

Parity status: every public function here is pinned by ``tests/test_oracle.py``
(brute force, closed forms, torch fp64 SDPA / autograd, finite differences and
the page's worked zig-zag example). No function is "parity unpinned".
"""

from .attention_fp64 import (  # noqa: F401
    CONTIGUOUS,
    ZIGZAG,
    accumulator_state,
    alibi_slopes,
    attention_rank_share,
    attention_rank_share_bwd,
    finalize_state,
    owner_rank,
    permute_from_ranks,
    permute_to_ranks,
    rank_positions,
    ring_schedule,
    visible_pairs,
)
from .rope_fp64 import inv_freq, rotary_embedding  # noqa: F401
