"""MI355X-native sparse MLA flash attention over a paged latent KV cache.

Submodules:
  sfa        -- thin ctypes binding over the C-ABI library ``libsfa.so`` (HIP kernels for gfx950)
  workloads  -- seeded synthetic input generators (random draws only; no attention arithmetic)

Nothing is imported eagerly: ``import mla_sparse_top_amd.sfa`` loads the native library and raises
if it has not been built.
"""

__all__ = ["sfa", "workloads"]
