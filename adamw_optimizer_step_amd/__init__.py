"""Hybrid Muon + AdamW optimizer step for MI355X (gfx950).

The computation runs in the hand-written HIP library ``libmuonadamw.so``
(C ABI: ``include/muon_adamw.h``); this package only marshals torch tensors
into it.  Build the library with ``python -m adamw_optimizer_step_amd.build``.
"""

from .api import (Plan, adamw_clip_step, expand_view, make_desc, make_hparams,  # noqa: F401
                  muon_momentum, muon_update, normuon_rownorm, ns_orthogonalize_batched,
                  ns_workspace_bytes, route)
from .optim import MuonAdamW  # noqa: F401
