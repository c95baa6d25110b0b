"""fp64 CPU oracle for the hybrid window-softmax + bidirectional delta-rule attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The HIP library never imports, links or calls it, and it shares no
code, header, table or constant with the HIP path: it is written from the
method's definition so that the two can be compared.

Source of the definition: the VDN-H3 article ("VDN-Minimax-H3", icman.com.cn
news 81972), its sections on the far field, the five steps of the
bidirectional linear branch, the update-rule table and the text state; and,
for the backward pass of the windowed softmax branch, the chain rule through
that softmax (``softmax_grad``), and for the linear branch's gradient the same
steps in torch float64 under autograd (``linear_grad``).

Every public function says which passage it follows and how it is pinned
(see ``tests/test_oracle_*.py``). No function here is "parity unpinned".
"""

from .hybrid_attn import (  # noqa: F401
    RULES,
    window_bounds,
    softmax_branch,
    softmax_rows,
    silu,
    l2_normalize,
    short_conv,
    features,
    frame_statistics,
    rule_step,
    frame_alpha,
    scan,
    gathered_state,
    readout,
    linear_branch,
    hybrid_attn_head,
    hybrid_attn,
    text_state,
    rel_frobenius,
)
from .softmax_grad import (  # noqa: F401
    softmax_lse,
    softmax_lse_rows,
    softmax_branch_grad,
    softmax_grad_rows,
)
from .linear_grad import linear_branch_torch, linear_branch_grad  # noqa: F401
from .block import rope_pairs, rope_angles, rope3d, block_fwd  # noqa: F401
from .routing import route_scores, route_keep, routed_softmax  # noqa: F401
