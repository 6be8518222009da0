"""MI355X-native exact attention (FlashAttention forward and backward).

The compute path is the HIP library ``libfa.so`` built from ``csrc/`` for
gfx950; :mod:`io_aware_tiled_fa_amd.binding` marshals torch tensors into its
C ABI.  Importing the package loads nothing; the binding loads the library on
first use and raises if it is missing.
"""

__all__ = ["forward", "backward", "bwd_workspace_size"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
