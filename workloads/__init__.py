"""Seeded synthetic particle workloads shared by the oracle tests, the GPU
tests and the benchmark.

This module only draws inputs (grid, positions, weights, magnetic field per
particle or on the grid nodes, species constants). It holds none of the
assembly arithmetic, so the oracle and the GPU path can both consume it
without sharing any of the method.

The workloads follow the isolation setup of Pennati & Markidis, "Mass Matrix
Assembly on Tensor Cores for Implicit Particle-In-Cell Methods" (Sec. 4.1):
a 3D periodic box, one species, a fixed number of particles per cell and
particles stored cell by cell. The named configurations extend it to two
species, shuffled order and a clustered density.
"""
from .gen import (Grid, Species, Case, WORKLOAD_NOTES, make_config, uniform_species, random_case,
                  clustered_counts, species_from_counts, grid_field, make_2d, positions_f32)

__all__ = ["Grid", "Species", "Case", "WORKLOAD_NOTES", "make_config", "uniform_species", "random_case",
           "clustered_counts", "species_from_counts", "grid_field", "make_2d", "positions_f32"]
