"""Float64 CPU oracle for the gated-delta-rule token mixer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

Every function is the plain definition written out, token by token, in
float64, following "On the Design of Qwen3.8-Next Architecture" as summarised
on the slinene ai-papers-daily page (Module A, Gated DeltaNet: the four-line
delta form of the recurrence and the output parameterisation) and on the
paper.rainbus.top digest (method step (1)); the front end (short causal
convolutions, SiLU, L2 normalisation and the gates) follows the
parameterisation block of the same Module A; multi-token (speculative)
decode is the same recurrence over a block of draft tokens, with a commit step
that advances the live state by the accepted prefix only; the backward is the
chain rule through the same recurrence, written out step by step in reverse.
The QSA indexer (key pooling, partial rotary embedding, block-causal ReLU
scores, top-K block selection) follows Module B of the same slinene page.
"""

from .gdn_ref import (  # noqa: F401
    gated_delta_recurrence,
    gated_delta_decode_step,
    gated_rmsnorm,
    rel_err,
)
from .frontend_ref import gdn_frontend, short_conv, silu, l2norm  # noqa: F401
from .mtp_ref import mtp_verify, mtp_commit  # noqa: F401
from .bwd_ref import gated_delta_backward  # noqa: F401
from .qsa_ref import rmsnorm, partial_rope, qsa_prep, qsa_scores, qsa_select, qsa_token_set  # noqa: F401
