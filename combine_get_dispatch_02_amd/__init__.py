"""MI355X-native MoE expert-parallel dispatch / combine.

The computation lives in libep.so (hand-written gfx950 HIP kernels behind the
C ABI of include/ep.h).  This package holds its thin Python binding
(:mod:`.ep`), the hipcc build step (:mod:`.build`) and the seeded synthetic
workload generator (:mod:`.workloads`).
"""
from .ep import (EPError, ep_combine, ep_dispatch, ep_dispatch_cached,  # noqa: F401
                 ep_dispatch_fp8, ep_dispatch_fp8_cached, ep_dispatch_ht,
                 ep_dispatch_ht_workspace_bytes, ep_dispatch_ll, ep_dispatch_ll_fp8,
                 ep_dispatch_ll_workspace_bytes, ep_dispatch_noalloc, ep_dispatch_workspace_bytes,
                 ep_get_dispatch_layout, ep_layout_workspace_bytes, lib, version)

__all__ = ["EPError", "ep_get_dispatch_layout", "ep_dispatch", "ep_dispatch_noalloc", "ep_dispatch_fp8",
           "ep_combine",
           "ep_dispatch_cached", "ep_dispatch_fp8_cached", "ep_dispatch_ht",
           "ep_dispatch_ht_workspace_bytes", "ep_dispatch_ll", "ep_dispatch_ll_fp8",
           "ep_dispatch_ll_workspace_bytes",
           "ep_layout_workspace_bytes", "ep_dispatch_workspace_bytes", "lib", "version"]
