"""MI355X-native gated delta rule (Gated DeltaNet / KDA): chunked prefill,
O(1)-state decode step and varlen packing with state snapshots, as hand-written
HIP kernels for gfx950 behind a C ABI (libkda.so, include/kda.h).

The binding in `kda` loads libkda.so on first use and raises if it is missing;
there is no CPU fallback."""
from .kda import (  # noqa: F401
    KDA_BF16, KDA_F32, KdaError, KdaShape, decode_step, decode_tokens, kda_abi_version, kda_decode_step, kda_decode_tokens,
    kda_last_error, kda_layer_back, kda_layer_front, kda_layer_prefill, kda_layer_prefill_workspace_size,
    kda_prefill_backward, kda_prefill_backward_workspace_size,
    kda_prefill_chunked, kda_prefill_chunked_noalloc, kda_prefill_workspace_size,
    kda_snapshot_count, layer_back, layer_front, layer_prefill, load, make_shape, prefill_backward, prefill_chunked)
from .autograd import gated_delta_rule  # noqa: F401,E402
