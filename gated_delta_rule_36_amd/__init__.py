"""Gated Delta Rule-2 token mixer for MI355X (gfx950): HIP kernels behind a C ABI.

    from gated_delta_rule_36_amd import chunk_fwd, decode_step

`chunk_fwd` runs the chunkwise-parallel forward over whole (optionally packed)
sequences, two-phase (with a workspace) or fused; `chunk_bwd` its gradients;
`decode_step` advances a pool of recurrent states by one token, `decode_tokens` by
several (with slot indexing and committed prefixes, for serving); `block_prologue` and
`block_epilogue` are the block's branches around the mixer. Both call libgdn2.so, built in-tree by
`python -m gated_delta_rule_36_amd.build`.
"""
from ._lib import (Gdn2Error, SavedForBackward, block_epilogue, block_prologue,
                   chunk_bwd, chunk_fwd, chunk_fwd_train, decode_step, decode_tokens,
                   gated_delta_rule2, lib, lib_path, uses_split, workspace_bytes)

__all__ = ["chunk_fwd", "chunk_fwd_train", "chunk_bwd", "gated_delta_rule2", "SavedForBackward",
           "decode_step", "decode_tokens", "block_prologue", "block_epilogue", "workspace_bytes",
           "uses_split", "lib", "lib_path", "Gdn2Error"]
