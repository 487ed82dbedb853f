"""fp64 CPU oracle of the Lighthouse attention layer (test infrastructure only;
see ``lighthouse_ref`` and ``layer_ref`` for what they compute and which
passages they follow)."""
from .lighthouse_ref import *  # noqa: F401,F403
from .lighthouse_ref import (attend, attend_adjoint, attend_rows, backward_head, budget, coords_of_flat,  # noqa: F401
                             flat_offsets, forward_head, from_fixed, gather, level_sizes,
                             order, pool_adjoint, pyramid, round_bf16, scatter, scatter_adjoint, scatter_fixed,
                             scatter_range, scores, select, subsequence_length_eq8, to_fixed,
                             window_end)
from .layer_ref import concat_heads, heads_of, layer_backward, layer_forward  # noqa: F401
