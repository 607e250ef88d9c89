"""MI355X (gfx950) verify-and-commit replay for Gated DeltaNet recurrent state.

The hot path is hand-written HIP in ``csrc/`` behind the C ABI of
``include/gdn_replay.h`` (plus an HBM bandwidth probe, ``include/gdn_probe.h``);
this package holds the ctypes binding (argument marshalling only), the in-tree
build script and the seeded workload generators.
"""
from ._binding import (  # noqa: F401
    EXPORTS, GDN_MAX_LAYERS, GDN_MAX_REC_TOKENS, GDN_PROBE_CHUNK, PROBE_COPY, PROBE_READ,
    PROBE_WRITE, RECORD_CHANNEL, RECORD_CORRECTION, RECORD_PAYLOAD, ConvPools, GdnError, Pools, ROW_BND, ROW_N,
    ROW_ALIAS, ROW_POS, ROW_REC, ROW_SLOT, ROW_TABLE, ROW_WIN, gdn_align_plan,
    gdn_commit_all_layers, gdn_bandwidth_probe, gdn_check_slots, gdn_commit_all_layers_conv, gdn_native_accept, gdn_native_window,
    gdn_verify, load_library, rec_stride,
)
