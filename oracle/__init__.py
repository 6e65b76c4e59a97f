"""CPU oracle for one tensor-parallel rank's share of the pre-RMSNorm MLP sublayer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``tensor_transformer_mlp_rmsnorm_amd``) never imports it, and this package
imports nothing from the GPU library: the two share no code.  Their only
common dependency is the seeded input module ``synth``, which holds no
arithmetic of the method.

The oracle is plain numpy, in float64 unless a caller asks for float32 (the
bf16 workloads state fp32 accumulation).  Matrix products use ``@`` as a
library primitive; everything else is written out as the pages define it.

Parity pins: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` (finite differences, autograd of a separately typed
block, closed forms, PyTorch library routines, the page's shape record and the
page's printed error magnitudes and ablation signatures).  None is unpinned.
"""

from .mlp import (  # noqa: F401
    Params,
    rms_norm_fwd,
    rms_norm_bwd,
    activation_fwd,
    activation_bwd,
    sigmoid,
    silu,
    silu_grad,
    gelu,
    gelu_grad,
    dense_step,
    sharded_step,
    fixture_record,
    inspect_record,
    row_forward_backward,
    MODES,
    bf16_round,
    storage_rounding,
)
from .sampled import sampled_step  # noqa: F401,E402
from .optim import (  # noqa: F401,E402
    ADAM_BETA1,
    ADAM_BETA2,
    ADAM_EPS,
    microbatch_bounds,
    accumulated_grads,
    global_grad_norm,
    clip_coefficient,
    adamw_update,
    adamw_step,
)
from .sequence import SP_MODES, sequence_parallel_step, sequence_slices  # noqa: F401,E402
from .fp8 import (  # noqa: F401,E402
    E4M3,
    E5M2,
    Fp8Meta,
    fp8_dense_step,
    fp8_sharded_step,
    new_metas as fp8_new_metas,
)
from .attention import (  # noqa: F401,E402
    ATTN_MODES,
    AttnParams,
    AttnShape,
    attn_dense_step,
    attn_sharded_step,
    causal_attention_fwd,
    causal_attention_bwd,
)
