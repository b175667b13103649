"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

Holds no attention arithmetic: see ``generate.py`` for the conventions.
"""
from .generate import (BLOCK_SIZE, HEAD_DIM, POISON, PagedWorkload, blocks_for,
                       build_workload, normal_bits)
from .configs import CONFIG_NAMES, DESCRIPTIONS, DEFAULT_SEEDS, make_config

__all__ = ["BLOCK_SIZE", "HEAD_DIM", "POISON", "PagedWorkload", "blocks_for", "build_workload",
           "normal_bits", "CONFIG_NAMES", "DESCRIPTIONS", "DEFAULT_SEEDS", "make_config"]
