"""Packed width-4 depthwise causal Conv1d (+ SiLU) for MI355X (gfx950)."""
