"""CPU oracle for HGA routed attention: TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP library and its binding.
"""
from .hga_oracle import (QueryRoute, attend, attend_tokens, build_summaries, dense_causal,
                         route, route_query, routed_tokens, score, top_k)
