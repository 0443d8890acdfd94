"""CPU oracle for RLA-2 causal ReLU linear attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path never does.
"""
from .rla2_oracle import (  # noqa: F401
    DEFAULT_EPS, DEFAULT_RMS_EPS, DEFAULT_ROPE_BASE,
    rms_norm, rope_frequencies, rope_rotate_half, feature_map, documents, first_documents,
    fwd, fwd_rows, fwd_recurrent, state_from_prefix, decode_step, decode_direct,
)
from .rla2_backward import fwd_torch, bwd, bwd_qk_prime, bwd_one_document, feature_map_torch  # noqa: F401,E402
from .rla_l2 import (DEFAULT_L2_EPS, fwd_l2, fwd_l2_rows, fwd_l2_recurrent, second_state_from_prefix,  # noqa: F401,E402
                     decode_step_l2)
