"""MI355X-native tree-attention verification pass.

The four calls of the pass (tree_mask_build, tree_attn_verify,
tree_accept_greedy, kv_compact_path) live in the HIP library
``libtreeverify.so`` behind a C ABI (include/treeverify.h); the Python binding
in ``binding`` only marshals arguments.  Importing this package loads nothing:
``binding`` loads the library on first use and fails loudly if it is missing.
"""
__all__ = ["workloads", "binding"]
