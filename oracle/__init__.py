"""CPU oracle (fp64 numpy) of partitioned DiT attention with selective state reuse.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with the HIP
path; both read their inputs from `workloads` (seeded draws and RoPE only).

Parity pins (see tests/test_oracle_pins.py and tests/test_oracle_planner.py):
  partition_state / merge_states  - full softmax attention by brute force; P = 1; closed
                                    forms (q = 0, constant V, equal keys); associativity
                                    and commutativity; merge weights sum to 1
  selective_step                  - closed form with q = 0 and constant V / V_prev;
                                    all-recompute == anchor; reuse of unchanged inputs
                                    == full attention
  importance                      - q = 0 closed form |p| / S_kv; sums to 1
  local_change                    - V_t = c V_{t-1} gives |c - 1|; unchanged gives 0
  RefPlanner                      - brute-force subset enumeration; round-robin closed
                                    form; hand-derived selection lists
  round_fp8_e4m3, fp8_store       - OCP e4m3 encodings of known values (ties to even,
                                    subnormals, the largest finite value); relative error
                                    of normals <= 2^-4
  decode_fp8_e4m3                 - known codes; every finite code is a fixed point of
                                    round_fp8_e4m3 and every rounded value is a code's value
                                    (two independent readings of the format agree)
  compose_states                  - composed state == brute-force attention over the union
                                    of the group's keys; merge after compose == merge;
                                    recursive composition == one-shot composition
"""
from .attention import (StateCache, StepResult, compose_states, full_attention, importance, local_change,
                        merge_states, merge_weights, partition_state, round_bf16, round_f32, round_fp8_e4m3,
                        fp8_store, decode_fp8_e4m3,
                        selective_step, block_of_rows)
from .planner import RefPlanner, group_distance, group_of
