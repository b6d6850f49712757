"""MI355X-native (gfx950) forward and backward of one tensor-parallel rank's
share of a Megatron-style Transformer block, plus the vocab-sharded
cross-entropy, behind a C-ABI library (``libmtb.so``).

``transformer_layer_ln_amd.mtb`` is the thin ctypes binding; importing this
package does not load the library.
"""
__all__ = ["inputs", "mtb"]
