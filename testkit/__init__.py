"""Seeded synthetic inputs shared by the oracle's tests, the GPU tests and the bench."""
from .gen import normal_f16, normal_f64
from .workloads import (CONFIGS, DECODE, HEADLINE, SPLITKV_BENCH, SWEEP, WORKLOADS, CacheWorkload,
                        Workload, cache_inputs, make_qkv, workload_inputs)

__all__ = ["normal_f16", "normal_f64", "CONFIGS", "DECODE", "HEADLINE", "SPLITKV_BENCH", "SWEEP",
           "WORKLOADS", "CacheWorkload", "Workload", "cache_inputs", "make_qkv", "workload_inputs"]
