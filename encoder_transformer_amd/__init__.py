"""MI355X-native forward pass of the Julia-1 decision model.

`encoder_transformer_amd.lib` binds the C-ABI library (``libjl.so``, built
from ``csrc/`` for gfx950); `encoder_transformer_amd.synth` draws seeded
weights and packed batches. Importing the package loads nothing.
"""
