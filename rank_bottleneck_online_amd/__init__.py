"""MI355X-native low-rank bottleneck block (Online-RMSNorm, grouped down
projection, SiLU/identity bottleneck, batched up projection, checkpointed
backward) behind a C-ABI HIP library.

The compute entry points live in :mod:`rank_bottleneck_online_amd.binding`
(loaded on first use so that the seeded input generator in
:mod:`rank_bottleneck_online_amd.synth` imports without the GPU library).
"""

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name == "binding":
        from . import binding
        return binding
    raise AttributeError(name)
