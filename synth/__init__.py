"""Seeded synthetic inputs for HGA routed attention (shared by the oracle's tests,
the GPU parity tests and the benchmark; holds none of the method's arithmetic)."""
from .workloads import Workload, ALL, TINY, TINY_ALL, DECODE_64K, SWEEP, PREFILL, HOST_TIER
from .inputs import Inputs, generate, gen_q, gen_kv_slice, plant_count, query_positions, round_to_dtype, rope
