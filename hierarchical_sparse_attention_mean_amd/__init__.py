"""MI355X-native Lighthouse attention (hierarchical sparse attention with mean
pooling) for one head-batch, forward and backward.

The compute path is the C-ABI library ``liblighthouse.so`` built from
``csrc/`` (hand-written HIP kernels for gfx950); ``lighthouse`` is its thin
ctypes binding and ``synth`` holds the seeded synthetic input generators.
Importing this package loads nothing; ``from hierarchical_sparse_attention_mean_amd
import lighthouse`` loads the library and fails loudly if it is not built.
"""
__all__ = ["lighthouse", "synth"]
