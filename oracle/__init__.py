"""Float64 CPU oracle for the RWKV-4 WKV operator, the token-shift mix, and the
matrix-state WKV of RWKV-5 and RWKV-6.

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.  See wkv_ref.py,
token_shift_ref.py, wkv5_ref.py and wkv6_ref.py for the sources each function follows and the readings
taken where the pages are silent.
"""
from .wkv_ref import (  # noqa: F401
    wkv_backward_ref,
    wkv_backward_state_ref,
    wkv_direct_ref,
    wkv_forward_ref,
    wkv_gated_backward_ref,
    wkv_gated_forward_ref,
    wkv_state_from_sums,
    wkv_state_grads_from_sums,
    wkv_step_ref,
    wkv_sums_from_state,
    wkv_sums_grads_from_state,
)
from .token_shift_ref import (  # noqa: F401
    shifted_inputs_ref,
    token_shift_backward_ref,
    token_shift_ref,
)
from .wkv5_ref import wkv5_backward_ref, wkv5_direct_ref, wkv5_forward_ref  # noqa: F401
from .wkv6_ref import wkv6_backward_ref, wkv6_direct_ref, wkv6_forward_ref  # noqa: F401
