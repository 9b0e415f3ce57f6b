"""Seeded synthetic workloads shared by the oracle tests, the GPU parity tests and the bench."""
from .synth import (TILE, Workload, config, make_workload, make_chunked_workload, chunk_legal_tiles,
                    cu_from_lengths, legal_tile_matrix,
                    route_bernoulli_groups, route_bernoulli_tiles, route_band_sink, fp32_inv_sqrt,
                    varlen_lengths, rng_for)

__all__ = ["TILE", "Workload", "config", "make_workload", "make_chunked_workload", "chunk_legal_tiles",
           "cu_from_lengths", "legal_tile_matrix",
           "route_bernoulli_groups", "route_bernoulli_tiles", "route_band_sink", "fp32_inv_sqrt",
           "varlen_lengths", "rng_for"]
