"""MI355X-native hybrid prefill/decode transformer-layer step.

The product is libhybrid_layer.so (C ABI in include/hybrid_layer.h, HIP kernels for gfx950 under
csrc/); `binding` exposes the same entry points to Python with torch tensors as device buffers.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    Batch, HLError, LayerCfg, alloc_workspace, attention, decode_attention, gemm_bf16_nt,
    hybrid_layer_step, layer_cfg, prefill_attention, qkv_rope_append, rms_scale, rmsnorm,
    rope_kv_append, strerror,
    workspace_bytes,
)
