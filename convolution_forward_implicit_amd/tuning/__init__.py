"""Tile-configuration selector calibration: sweep.py times every compiled
configuration on a grid of problems (GPU), fit.py fits the per-configuration
cost model from that table and writes the coefficients the library's
selector uses (csrc/selector_coef.inc)."""
