"""Seeded synthetic workloads shared by the CPU oracle and the GPU library's tests.

Only shapes, seeds and random draws live here; no decoder arithmetic.
"""
from .configs import (BF16, F32, LLAMA_1B, LLAMA_8B, LLAMA_LAYER_F32, QWEN_8B, ModelConfig,
                      Plan, RunConfig, Workload, WORKLOADS, shrink)
from . import gen

__all__ = ["BF16", "F32", "LLAMA_1B", "LLAMA_8B", "LLAMA_LAYER_F32", "QWEN_8B", "ModelConfig",
           "Plan", "RunConfig", "Workload", "WORKLOADS", "shrink", "gen"]
