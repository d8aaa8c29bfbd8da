"""LTX-2 per-block attention set (video self, audio self, a2v, v2a) on MI355X.

* ``ltxattn`` -- binding of the C ABI of ``libltxattn.so`` (HIP kernels).
* ``synth``   -- seeded synthetic bf16 inputs of the measured workloads.
* ``build``   -- compiles the library in-tree for gfx950.

Importing the package loads nothing; ``from video_audio_diffusion_ltxattn_amd
import ltxattn`` loads the library and fails loudly if it is not built.
"""
