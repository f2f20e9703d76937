"""MI355X-native IO-aware exact attention (forward and backward) behind a C-ABI library.

The HIP kernels live in ``csrc/`` and are built into ``libfa.so`` by
``exact_attention_110_amd.build``; ``binding`` calls them through ctypes with
torch tensors for memory and the current stream; ``inputs`` draws the seeded
synthetic workloads.
"""

_API = ("forward", "backward", "backward_stage", "workspace", "workspace_size", "status_string", "FAError")


def __getattr__(name):
    if name in _API:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
