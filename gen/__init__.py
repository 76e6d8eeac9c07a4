"""Seeded synthetic input generators (no method arithmetic)."""
from .synth import *  # noqa: F401,F403
from .synth import CONFIGS, CFG1, CFG2, CFG3, CFG4, CFG5, CFG_FP8  # noqa: F401
