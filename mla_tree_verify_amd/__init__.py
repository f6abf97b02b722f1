"""MLA tree-verify attention for MI355X (gfx950): HIP kernels behind a C ABI.

    from mla_tree_verify_amd import mla_verify
    out, lse = mla_verify(q_nope, q_rope, kv_latent, k_rope, tree_parent, prefix_len, scale)

The library (libmla_verify.so, built by `python -m mla_tree_verify_amd.build`)
is loaded on first use; there is no CPU fallback.
"""
_API = ("mla_verify", "mla_verify_batched", "mla_verify_partials", "combine", "device_plan")


def __getattr__(name):
    if name in _API:
        from . import api

        return getattr(api, name)
    raise AttributeError(name)
