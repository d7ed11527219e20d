"""Causal kernelized linear attention ("Transformers are RNNs") on MI355X.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI of
liblinattn.so (include/linattn.h).  This package is the thin Python binding:
argument marshalling only; PyTorch supplies device memory and streams.
"""
from .features import draw_projection  # noqa: F401
from .linattn import (  # noqa: F401
    LinAttnError,
    backward,
    decode_step,
    decode_step_features,
    decode_steps,
    feature_map,
    feature_map_backward,
    forward_chunked,
    forward_chunked_noalloc,
    forward_continue,
    forward_features,
    forward_fused,
    forward_onepass,
    forward_plan,
    probe_copy,
    probe_mfma,
    probe_read,
    probe_write,
    fused_workspace_bytes,
    lib_path,
    noalloc_scratch_bytes,
    segment_outputs,
    segment_scan,
    segment_states,
    softmax_scan,
    softmax_step,
    version,
    workspace_bytes,
    workspace_init,
    workspace_status,
)
