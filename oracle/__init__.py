"""CPU oracle for the online-softmax row kernel and the fused attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything in this package: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, and by nothing else.

Every function here is a plain, slow, float64 restatement of the definitions on
the source pages:

* "Ch.6 Softmax and Online Softmax" (yangyitao.com, the CUDA FlashAttention-v2
  book), cited below as [Ch6 §x];
* the xxqk.cn article on parallelising softmax, Online Softmax and
  FlashAttention, cited as [xxqk §x];
* the mooersco.com article "FlashAttention 2.0 in LLM inference", cited as
  [mooers §x].

Modules
-------
softmax_ref    three-pass safe softmax ([Ch6 §6.2]), its fused additive-mask /
               row-length form ([Ch6 §6.7.3]), and the unsafe two-pass form
               ([Ch6 §6.1]) kept as a negative control.
online_ref     the element-wise online normaliser and the (m, l) combine
               ([Ch6 §6.3.1], [Ch6 §6.4.1]); used only to check the oracle
               itself (online == two-pass by brute force).
attention_ref  materialised-S attention with log-sum-exp ([Ch6 §6.5],
               [Ch6 §6.6], [xxqk §4.2]) and the single-query blocked alpha/beta
               form ([Ch6 §6.6]) as a self-check.
attention_bwd_ref
               gradients dQ, dK, dV of that attention through the softmax
               Jacobian (the backward that [Ch6 §6.5] and [xxqk §5.2] say
               recomputes S from the saved log-sum-exp).

The oracle shares no code with the HIP library and never imports it.  Pins that
tie it to something other than itself live in ``tests/test_oracle_*.py``.
Parity status of each function is stated in its docstring.
"""

from .softmax_ref import masked_softmax_rows_ref, naive_softmax_rows_f32, softmax_rows_ref
from .online_ref import EMPTY_STATE, all_trees, combine, online_state, singleton, tree_reduce
from .attention_ref import attention_head_ref, attention_ref, blocked_attention_row_ref
from .attention_bwd_ref import (attention_bwd_head_ref, attention_bwd_ref, attention_dq_rows_ref,
                                attention_probs_head_ref)

__all__ = [
    "softmax_rows_ref",
    "masked_softmax_rows_ref",
    "naive_softmax_rows_f32",
    "EMPTY_STATE",
    "combine",
    "singleton",
    "online_state",
    "tree_reduce",
    "all_trees",
    "attention_head_ref",
    "attention_ref",
    "blocked_attention_row_ref",
    "attention_probs_head_ref",
    "attention_bwd_head_ref",
    "attention_bwd_ref",
    "attention_dq_rows_ref",
]
