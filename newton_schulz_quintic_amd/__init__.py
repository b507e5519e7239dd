"""MI355X (gfx950) Newton-Schulz orthogonalisation with shard routing.

The work happens in the HIP library ``libnsq.so`` behind the C ABI of
``include/ns.h``; this package is its ctypes binding (``_lib``) plus the
in-tree build (``build``). Importing the package does not load the library;
the first call does, and fails loudly if it was never built.
"""

from ._lib import (  # noqa: F401
    NS_BF16,
    NS_F32,
    NS_MAX_SHARDS,
    EXPORTS,
    LIB_PATH,
    NSError,
    NSLibraryMissing,
    RoutePlan,
    lib,
    ns_last_error,
    ns_gram_workspace_bytes,
    ns_noalloc_init,
    ns_orthogonalize_batched,
    ns_orthogonalize_batched_noalloc,
    ns_orthogonalize_gram,
    ns_orthogonalize_routed,
    ns_orthogonalize_strided,
    ns_orthogonalize_waves,
    ns_pack_shards,
    ns_plan,
    ns_route_plan_create,
    ns_route_plan_create_axis,
    ns_route_plan_destroy,
    ns_route_plan_query,
    ns_route_plan_upload,
    ns_timing_enable,
    ns_timing_read,
    ns_unpack_shards,
    ns_version,
    ns_wave_plan,
    ns_routed_workspace_bytes,
    ns_workspace_bytes,
)
