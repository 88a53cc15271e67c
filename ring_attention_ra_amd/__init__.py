"""One ring rank's share of causal blockwise attention on MI355X (gfx950).

The work runs in libra.so (HIP kernels behind a C ABI, see include/ra.h);
``_lib`` binds its entry points one to one and ``ring`` sequences them as the
chunks one rank receives around a simulated ring.
"""

from . import configs  # noqa: F401
from ._lib import (  # noqa: F401
    RaError,
    ra_abi_version,
    ra_bwd_delta,
    ra_count_nonfinite,
    ra_finalize,
    ra_last_error,
    ra_layout_permute,
    ra_positions,
    ra_state_init,
    ra_step_bwd,
    ra_step_fwd,
)
from .ring import alibi_slopes, backward, forward, positions, ring_schedule, shard  # noqa: F401
