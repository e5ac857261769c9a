"""MI355X-native fine-grained MoE layer (routing with token rounding,
gather-fused grouped GEMMs, minimal-activation backward).

The HIP library is loaded on first use by :mod:`fine_grained_mixture_amd.moe`.
"""
