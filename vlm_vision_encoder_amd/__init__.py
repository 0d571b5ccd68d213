"""MI355X-native Pixtral-class vision tower.

The compute path is the HIP library ``libpv_tower.so`` (C ABI declared in
``include/pv_tower.h``); ``vlm_vision_encoder_amd.tower`` is its thin ctypes
binding.  ``vlm_vision_encoder_amd.synth`` makes seeded synthetic inputs.
Importing the package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""
__all__ = ["tower", "synth"]
