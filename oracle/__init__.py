"""fp64 CPU oracle of DARKFormer PRF attention: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP library and never calls it.
"""
from .omega_gen import (  # noqa: F401
    head_seed,
    normals,
    omega,
    omega_iid,
    omega_orthogonal,
    omega_per_head,
    splitmix64,
    uniforms,
)
from .prf_oracle import (  # noqa: F401
    attend_causal_blockwise,
    attend_noncausal,
    attention,
    attention_backward,
    attention_backward_noncausal_head,
    context_state,
    cross_attention,
    decode_step,
    exact_kernel_attention,
    head_geometry,
    head_omega,
    kv_head,
    prf_features,
    project,
    qk_scale,
)
