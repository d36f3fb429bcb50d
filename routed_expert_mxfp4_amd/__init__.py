"""routed_expert_mxfp4_amd: one routed MoE FFN layer (top-k of E experts,
MXFP4 experts) as a C-ABI HIP library for gfx950, with a thin Python binding.

Importing the package loads nothing; ``routed_expert_mxfp4_amd.moe`` loads the
compiled library on first use and raises if it is missing.
"""
__all__ = ["synth", "moe"]
