"""chunk_wise_causal_amd — the chunk-wise causal attention hot path of
streaming video diffusion ("Wave Forcing: Towards Speed-of-Light Streaming
Video Generation", §3.1 and §4.2) as a gfx950-native C-ABI library, libwf.

The C ABI (include/wf.h) has two calls, wf_kv_publish and wf_chunk_attn; the
binding in chunk_wise_causal_amd.wf mirrors them with torch tensors standing
in for device pointers.  Importing the package does not load the library; the
first call does, and raises if libwf.so is missing.
"""
__version__ = "0.1.0"


def __getattr__(name):
    if name in ("KVPool", "wf_kv_publish", "wf_chunk_attn", "wf_device_status",
                "WFError", "lib"):
        import importlib
        return getattr(importlib.import_module(__name__ + ".wf"), name)
    raise AttributeError(name)
