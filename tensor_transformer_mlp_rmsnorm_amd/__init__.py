"""One tensor-parallel rank's share of the pre-RMSNorm MLP sublayer on MI355X.

The compute lives in ``libtpmlp.so`` (HIP kernels for gfx950 behind the C
ABI of ``include/tp_mlp.h``).  ``_lib`` binds its entry points under the same
names (import them from there); ``step`` sequences them over the shards of one
training step.
Importing this package does not load the library; the first call does, and
raises if it has not been built.
"""
