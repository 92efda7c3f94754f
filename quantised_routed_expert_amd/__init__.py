"""MI355X (gfx950) routed-expert MoE layer: exact router, fused SMOE-Q4 /
SMOE-Q2 expert FFN for decode, layer-major prefill with a per-chunk expert
union, and an LRU expert ring.  The computation lives in the HIP library libsmoe.so; this package
only binds it (see include/smoe.h for the C ABI)."""
from .binding import (SmoeError, Ring, blob_bytes, blob_stride, workspace_bytes, workspace, route, route_ext,
                      moe_decode, moe_decode_slots, decode_layers, decode_layers_static, moe_prefill_chunk, lib, dims_struct,
                      PinnedHost, EXPORTED, LIB_PATH)
