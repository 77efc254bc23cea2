"""Microbenchmarks of the gfx950 issue limits that bound the bdattn kernels."""
