"""MI355X-native multi-scale deformable attention (MSDeformAttn) core.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI
of include/msda.h (libmsda.so, built in-tree by ``build.py``).  The entry
points below load that library on first use and raise ImportError if it has
not been built; there is no other implementation to fall back to.
"""

_OPS = ("MSDeformAttnFunction", "ms_deform_attn", "forward", "backward", "problem_for",
        "MSDeformAttnFusedFunction", "ms_deform_attn_fused", "forward_fused", "backward_fused")


def __getattr__(name):
    if name in _OPS:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
