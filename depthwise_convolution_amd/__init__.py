"""Depthwise 2-D convolution for MI355X (gfx950): binding to the HIP library."""
