"""MI355X (gfx950) MLA latent-KV attention: C-ABI HIP library + thin binding.

Importing the package does not load the shared library; `mla_latent_kv_24_amd.api`
does, and raises if it is missing.
"""
