"""Plain fp64 CPU oracle for the tiled-attention hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call, link
or execute anything under ``oracle/``. The only permitted users are the test
suite (``tests/``), ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``. The oracle shares no code, constants or helpers with the HIP
library in ``attention_fa2_tiles_amd/``; it receives the same seeded inputs
(already rounded to the storage dtype, upcast to float64) and computes each
result straight from its definition with numpy float64.

Contents
--------
attention.py
    ``attn_fwd``, ``attn_bwd``, ``attn_fwd_jvp``, ``pw_fwd``, ``pw_bwd`` and
    the masks they use.  Sources: the Triton fused-attention tutorial with JVP
    support (Birch-san's gist ``_06_fused_attention_blockptr_jvp.py`` and its
    comment thread) and FlagAttention ``src/flag_attn/piecewise.py``.
merge.py
    ``merge_fwd`` and ``merge_bwd`` for the block-residual two-way
    online-softmax merge; ``lse_merge_fwd`` and ``lse_merge_bwd``, its N-way
    form with given logits (the merge of attention partials).  Source: flash_attn_res 0.1.11,
    ``slop/backward_phase_2.txt`` (``reference_forward`` and the phase-2 merge
    backward kernel).

Every function here is pinned by a CPU test in ``tests/test_oracle_*.py``
against something other than itself (a library routine, brute force,
finite differences, closed forms or invariants).  No function is left
"parity unpinned".
"""

from .attention import (  # noqa: F401
    allowed_mask,
    near_mask,
    attn_probs,
    attn_fwd,
    attn_bwd,
    attn_fwd_jvp,
    pw_fwd,
    pw_bwd,
)
from .merge import merge_fwd, merge_bwd, lse_merge_fwd, lse_merge_bwd  # noqa: F401
