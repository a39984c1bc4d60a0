"""CPU fp64 oracle for the Mamba-2 SSD forward pass.

This package is TEST INFRASTRUCTURE. Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run it. The product path (the HIP library and its Python binding)
never imports it, and it imports nothing from the product path.

Contents (all in ``oracle.ssd_oracle``):

* ``ssd_recurrent``    -- the plain sequential recurrence: the definition.
* ``ssd_quadratic``    -- the masked-attention (dual) form of the same matrix.
* ``ssd_semiseparable_matrix`` -- the explicit semiseparable matrix, for brute
  force on tiny inputs.
* ``ssd_chunked``      -- the blocked two-pass algorithm (chunks, then
  recombined per-chunk states), independent code used only as a pin.
* ``chunk_cumsum``, ``chunk_local_states``, ``chunk_entry_states`` -- the
  intermediate quantities each step of the chunked path produces, computed
  from their plain definitions, for per-step parity.
* ``dt_preprocess``    -- the optional dt transformation (bias, softplus,
  clamp) applied before the recurrence.
* ``causal_conv1d``    -- the short causal convolution in front of the SSM.

Every function is pinned by ``tests/test_oracle_pins.py``.
"""

from .ssd_oracle import (  # noqa: F401
    ssd_recurrent,
    ssd_quadratic,
    ssd_semiseparable_matrix,
    ssd_chunked,
    chunk_cumsum,
    chunk_local_states,
    chunk_entry_states,
    group_of_head,
    dt_preprocess,
    causal_conv1d,
)
