"""CPU oracle for the Pixtral-class vision tower.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
reference that the HIP path is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with ``vlm_vision_encoder_amd`` and imports
nothing from it; both sides receive the same seeded arrays from
``vlm_vision_encoder_amd.synth`` (which holds no tower arithmetic).

Everything is computed in float64 with numpy.  See ``pv_oracle`` for the
functions and the passage of the pages each one follows.
"""
from .pv_oracle import (  # noqa: F401
    TowerConfig,
    plan_maps,
    patch_embed,
    rms_norm,
    rope_omega,
    rope_2d,
    attention,
    swiglu_mlp,
    merge_project,
    tower_forward,
)
