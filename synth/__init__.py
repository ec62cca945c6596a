"""Seeded synthetic inputs shared by the oracle and the HIP path (no method arithmetic)."""
from .workloads import (CONFIGS, DECODE_7B, MIXED_13B, MLP_70B, PREFILL_7B, TINY, Spec,
                        Workload, adapter_pages_per_class, generate, small_spec)

__all__ = ["CONFIGS", "TINY", "DECODE_7B", "PREFILL_7B", "MIXED_13B", "MLP_70B", "Spec",
           "Workload", "generate", "small_spec", "adapter_pages_per_class"]
