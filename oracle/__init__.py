"""CPU oracle for the Newton-Schulz hot path: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (``newton_schulz_quintic_amd``), and the HIP library never imports it.

Sources followed (web pages; cited by page title and section):

* "core.distributed.fsdp.src.megatron_fsdp.experimental.owner_planning"
  (Megatron-FSDP API docs): ``select_ge_2d_params``, ``ns_cost_fn``,
  ``_OwnerWork``, ``assign_owner_work``, ``OwnerGatherPlan`` (its worked
  example), ``OwnerScatterPlan``.
* "core.optimizer.layer_sharded_a2a" (Megatron Core API docs):
  ``params_by_home``, ``route_to_ns_home``, ``route_from_ns_home``.
* "[GTP][Muon] Optimize Muon step performance" (GitHub issue): the
  bitwise-parity requirement under "Current Progress".

Modules:

* :mod:`oracle.planner` -- eligibility, matrix view, cost, LPT owner
  assignment, ``params_by_home``, route offsets. Python integers.
* :mod:`oracle.route`   -- pack (gather shards to homes) and unpack (scatter
  results back to shards). NumPy slicing and concatenation, bit copies.
* :mod:`oracle.ns`      -- Newton-Schulz in float64 (NumPy matmul).

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (hand values from the pages, closed forms, brute force); the pin
for each function is named in its docstring.
"""
