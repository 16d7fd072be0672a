"""MI355X-native low-rank bottleneck block (Online-RMSNorm, grouped down
projection, SiLU/identity bottleneck, batched up projection, checkpointed
backward) behind a C-ABI HIP library.

The compute entry points live in :mod:`rank_bottleneck_online_amd.binding`
(import it explicitly; it needs torch and the built library), the seeded
input generator in :mod:`rank_bottleneck_online_amd.synth`.
"""
