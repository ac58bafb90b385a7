"""CPU oracle for block-sparse / top-k-selected attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``top_selected_attention_amd``) never imports it, and this package
imports nothing from the product path: the two share no code.

Everything here is plain numpy in float64: inputs are upcast exactly from
bf16/fp16, the score matrix S and the probability matrix P are materialised
explicitly over the selected keys, and gradients are scatter-added back.  No
blocking, fusion or online softmax: each function is the definition it cites,
written out.

Sources (the pages are CANN operator documents and one news page):

* "aclnnBlockSparseAttentionGrad", formula section: the forward
  ``Softmax(Mask(scale * query * key_sparse^T, atten_mask)) * value_sparse`` and
  the backward chain softmax_grad, dP, dS, dV, dQ, dK.
* "aclnnNsaSelectedAttention", formulas section: the Gather of key/value rows by
  ``topk_indices`` followed by masked softmax attention; constraints section
  for sparseMode 0/2.
* "aclnnSparseFlashAttention", formulas and constraints sections:
  ``softmax(Q K~^T / sqrt(d_k)) V~`` over the selected K~/V~, D = 512 plus a
  64-wide rope part.
* "SparseAttnSharedkvMetadata" (news page), parameter list: cu_seqlens as B+1
  prefix sums, seqused_kv, rightDownCausal mask mode 3.
* "aclnnFusedFloydAttentionGrad", formula section: scores as the sum of two
  products batched over different sequence axes, one softmax, and its
  backward chain (module ``floyd``).

Parity status per function is stated in each module's header.
"""

from .attention import (  # noqa: F401
    attend_fwd,
    attend_bwd,
    bsa_fwd,
    bsa_bwd,
    bsa_fwd_tnd,
    bsa_bwd_tnd,
    bsa_keys,
    nsa_fwd,
    nsa_bwd,
    nsa_keys,
    sfa_fwd,
    sfa_fwd_tnd,
    sfa_sharedkv_fwd,
)
from .compaction import bsa_compact, nsa_compact  # noqa: F401
from .floyd import floyd_fwd, floyd_bwd  # noqa: F401
