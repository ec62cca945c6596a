"""fp64 CPU oracle of the LoRA delta (test infrastructure; see slora_oracle's header)."""
from .slora_oracle import (AdapterEntry, AllocatorModel, OracleError, OracleState, PoolImage,
                           Segments, build_from_workload, lora_delta, lora_forward, round_to,
                           segment_model, workload_delta, workload_forward)

__all__ = ["AdapterEntry", "AllocatorModel", "OracleError", "OracleState", "PoolImage",
           "Segments", "build_from_workload", "lora_delta", "lora_forward", "round_to",
           "segment_model", "workload_delta", "workload_forward"]
