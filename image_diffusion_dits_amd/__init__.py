"""MI355X-native RainFusion2.0 online block-sparse attention.

The hot path lives in the C-ABI library built from ``csrc/`` (HIP for
gfx950); ``image_diffusion_dits_amd.rf`` is its thin Python binding.
"""
