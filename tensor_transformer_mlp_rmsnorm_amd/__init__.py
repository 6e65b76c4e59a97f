"""One tensor-parallel rank's share of the pre-RMSNorm MLP sublayer on MI355X.

The compute lives in ``libtpmlp.so`` (HIP kernels for gfx950 behind the C
ABI of ``include/tp_mlp.h``).  ``_lib`` binds its entry points under the same
names; ``step`` sequences them over the shards of one training step.
Importing this package does not load the library; the first call does, and
raises if it has not been built.
"""

from ._lib import (  # noqa: F401
    TPMLPError,
    tp_mlp_forward,
    tp_partial_sum,
    tp_rmsnorm_forward,
    tp_mlp_backward,
    tp_mlp_workspace_bytes,
    tp_mlp_sgd_step,
    tp_mlp_sgd_step_multi,
    tp_mlp_adamw_step_multi,
    tp_mlp_clip_grad_norm,
    tp_mlp_clip_grad_norm_workspace_bytes,
    make_adamw_hparams,
    tp_mlp_last_error,
    tp_mlp_version,
    make_desc,
)

__all__ = [
    "TPMLPError", "tp_mlp_forward", "tp_partial_sum", "tp_rmsnorm_forward", "tp_mlp_backward", "tp_mlp_workspace_bytes",
    "tp_mlp_sgd_step", "tp_mlp_sgd_step_multi", "tp_mlp_adamw_step_multi", "tp_mlp_clip_grad_norm",
    "tp_mlp_clip_grad_norm_workspace_bytes", "make_adamw_hparams", "tp_mlp_last_error", "tp_mlp_version",
    "make_desc",
]
