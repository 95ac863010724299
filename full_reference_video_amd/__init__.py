"""MI355X-native per-frame float_ssim and MS-SSIM scoring.

The scoring runs in the HIP library ``libvqm.so`` behind a C ABI
(``include/vqm.h``); ``full_reference_video_amd.vqm`` is its thin ctypes
binding.  ``full_reference_video_amd.synth`` draws the seeded synthetic frames.
Importing the package loads nothing native: the binding loads the library on
first use and raises if it is missing.
"""

__all__ = ["synth", "vqm"]
