"""Seeded synthetic workloads (shapes and input generators); no codec arithmetic."""
from .configs import ALL, BY_NAME, Workload, TINY, LLAMA8B_4BIT, QWEN7B_2BIT, LLAMA8B_LONG, PERHEAD_R6
from . import generators
