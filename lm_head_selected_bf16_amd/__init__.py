"""Fused linear selected-token log-probability for AMD MI355X (gfx950).

    logp = log_softmax((hidden @ W^T + b) / T)[target]     (0 for out-of-range targets)

and its backward to hidden, W and b, computed by hand-written HIP kernels in
libflp.so behind the C ABI of include/flp.h.  This package holds the build
script, the ctypes binding (same names as the C ABI) and a thin PyTorch
wrapper with autograd.

Also behind the same ABI: the vocabulary-shard partial forward and its merge
(forward_partial, merge), the operator on materialised logits (logits_logp,
logits_forward, logits_backward), the indexed row-subset variants of both
operators (linear_logp_indexed, logits_logp_indexed, ...), the untied embedding
lookup with its deterministic grad_weight (embedding), and measurement probes
(flp_probe_mfma, flp_probe_read).
"""
from ._abi import (FLP_BF16, FLP_F16, FLP_F32, FLP_I32, FLP_I64, FLP_OK, FlpError,  # noqa: F401
                   flp_backward, flp_backward_chunk_rows, flp_backward_indexed,
                   flp_backward_indexed_workspace_bytes,
                   flp_backward_workspace_bytes, flp_build_info, flp_embedding_backward,
                   flp_embedding_backward_workspace_bytes, flp_embedding_forward, flp_forward,
                   flp_forward_indexed, flp_forward_noalloc, FLP_FORWARD_NOALLOC_MAX_BYTES,
                   flp_forward_indexed_workspace_bytes, flp_forward_partial,
                   flp_forward_partial_bytes, flp_forward_workspace_bytes, flp_logits_backward,
                   flp_logits_backward_indexed, flp_logits_forward, flp_logits_forward_indexed,
                   flp_logits_indexed_workspace_bytes, flp_merge, flp_probe_mfma, flp_probe_read,
                   flp_probe_scratch_bytes, flp_profile_enable,
                   flp_profile_read, flp_status_string, load)
from .torch_ops import (LinearLogp, backward, backward_workspace_bytes,  # noqa: F401
                        LogitsLogp, default_backward_workspace_bytes, forward, forward_partial,
                        linear_logp, linear_logp_with_lse, logits_backward, logits_forward,
                        logits_logp, merge, LinearLogpIndexed, LogitsLogpIndexed,
                        backward_indexed, forward_indexed, linear_logp_indexed,
                        logits_backward_indexed, logits_forward_indexed, logits_logp_indexed,
                        Embedding, embedding, embedding_backward, embedding_forward)

__all__ = [
    "FLP_BF16", "FLP_F16", "FLP_F32", "FLP_I32", "FLP_I64", "FLP_OK", "FlpError",
    "flp_forward", "flp_backward", "flp_forward_workspace_bytes", "flp_backward_workspace_bytes",
    "flp_forward_noalloc", "FLP_FORWARD_NOALLOC_MAX_BYTES",
    "flp_backward_chunk_rows",
    "flp_forward_partial", "flp_forward_partial_bytes", "flp_merge",
    "flp_logits_forward", "flp_logits_backward",
    "flp_forward_indexed", "flp_forward_indexed_workspace_bytes", "flp_backward_indexed",
    "flp_backward_indexed_workspace_bytes", "flp_logits_forward_indexed",
    "flp_logits_backward_indexed", "flp_logits_indexed_workspace_bytes",
    "flp_embedding_forward", "flp_embedding_backward", "flp_embedding_backward_workspace_bytes",
    "flp_probe_scratch_bytes", "flp_probe_mfma", "flp_probe_read",
    "flp_status_string", "flp_build_info", "flp_profile_enable", "flp_profile_read", "load",
    "LinearLogp", "forward", "backward", "backward_workspace_bytes",
    "default_backward_workspace_bytes", "linear_logp", "linear_logp_with_lse",
    "forward_partial", "merge",
    "LogitsLogp", "logits_forward", "logits_backward", "logits_logp",
    "LinearLogpIndexed", "forward_indexed", "backward_indexed", "linear_logp_indexed",
    "LogitsLogpIndexed", "logits_forward_indexed", "logits_backward_indexed",
    "logits_logp_indexed",
    "Embedding", "embedding", "embedding_forward", "embedding_backward",
]
