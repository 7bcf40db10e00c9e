"""MI355X-native gated delta rule (Gated DeltaNet / KDA): chunked prefill,
O(1)-state decode step and varlen packing with state snapshots, as hand-written
HIP kernels for gfx950 behind a C ABI (libkda.so)."""
