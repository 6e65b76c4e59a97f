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
    MODES,
    Params,
    activation_bwd,
    activation_fwd,
    bf16_round,
    dense_step,
    fixture_record,
    gelu,
    gelu_grad,
    inspect_record,
    rms_norm_bwd,
    rms_norm_fwd,
    row_forward_backward,
    sharded_step,
    sigmoid,
    silu,
    silu_grad,
    storage_rounding,
)
from .sampled import sampled_step  # noqa: F401,E402
from .optim import (  # noqa: F401,E402
    ADAM_BETA1,
    ADAM_BETA2,
    accumulated_grads,
    adamw_step,
    adamw_update,
    clip_coefficient,
    global_grad_norm,
    microbatch_bounds,
)
from .sequence import sequence_parallel_step  # noqa: F401,E402
from .fp8 import fp8_dense_step  # noqa: F401,E402
from .attention import attn_dense_step, attn_sharded_step  # noqa: F401,E402
