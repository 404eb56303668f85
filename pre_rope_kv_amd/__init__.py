"""pre_rope_kv_amd: pre-RoPE KV injection with Chunked RoPE on MI355X (gfx950).

The compute path lives in the native library ``libprkv.so`` (C ABI, declared in
``include/prkv.h``): a host-side store and slot-mapping builder in C++, and one
HIP inject kernel that gathers pre-RoPE K/V rows, rotates K to serving-time
positions and scatter-copies K and V into a paged KV cache.

``pre_rope_kv_amd.prkv`` is the thin ctypes binding (same names as the C ABI).
It is imported lazily so that input generation works without the library; any
call into the binding raises if ``libprkv.so`` has not been built.
"""

__all__ = ["prkv", "workloads"]
