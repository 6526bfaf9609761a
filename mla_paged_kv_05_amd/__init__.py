"""MI355X-native paged MLA decoding: gfx950 HIP kernels behind a C ABI
(include/mla.h, libmla.so) with a thin ctypes binding.

The binding is imported lazily so that the seeded workload generators
(``mla_paged_kv_05_amd.workloads``) can be used without the HIP library.
"""
__all__ = ["get_mla_metadata", "mla_decode_with_kvcache", "mla_decode_noalloc", "num_sched_slots", "workspace_bytes",
           "debug_gather", "MlaError", "load_library", "PIECE_COST_FUSED"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
