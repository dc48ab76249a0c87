"""Absorbed-MLA decode and latent-cache append for MI355X (gfx950).

The compute path is the HIP library ``libmla.so`` (C ABI in ``include/mla.h``);
``mla_latent_kv_06_amd.binding`` marshals torch tensors into it.  Importing the
package itself loads nothing: ``from mla_latent_kv_06_amd import binding``
loads the library and fails loudly if it has not been built.
"""
