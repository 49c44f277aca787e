"""Sparse MLA forward over fp8_ds_mla records for MI355X (gfx950).

The compute path is libsmla.so (hand-written HIP kernels behind the C ABI in
include/smla.h); ``binding`` is its thin Python binding.  The binding is
imported on first use of any public name, and raises ImportError there if the
library has not been built (``python -m sparse_mla_decode_fp8_amd.build``):
there is no fallback path.
"""

_PUBLIC = (
    "MAX_HEADS", "MAX_SPLIT", "KernelTimer", "KvPool", "SmlaError", "cache_write", "decode_rows", "qk_probe", "fwd",
    "fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "fwd_paged", "fwd_v41", "v41_workspace_bytes", "mxfp8",
    "set_option", "split_for", "supported", "workspace", "workspace_bytes", "LIB_PATH", "EXPORTED",
)

__all__ = list(_PUBLIC)


def __getattr__(name):
    if name in _PUBLIC:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
