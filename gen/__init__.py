"""Seeded synthetic input generators shared by the oracle-side and GPU-side tests."""
from .synth import CONFIGS, LayerConfig, make_layer, make_scores, make_w, make_x  # noqa: F401
