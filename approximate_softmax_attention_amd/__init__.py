"""MI355X-native (gfx950) HyperAttention: near-linear approximate softmax
attention with a sortLSH hash, sampled row sums and V-norm-sampled products,
and a causal halving recursion, forward and backward, behind a C ABI
(include/hyperattn.h).

The torch-facing binding lives in ``api``; ``workloads`` makes the seeded
synthetic inputs. Importing the package does not load the HIP library; the
first call into ``api`` does, and fails if it has not been built.
"""

__all__ = ["api", "workloads"]
