"""CPU oracle for the cross-layer MoE step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct CPU implementation of what the GPU path
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product library never
calls it, and it imports nothing from the product library (or from the shared
input generators): it takes numpy arrays and returns numpy arrays.

Sources (the method's pages):

* [PAPER] "EasyBalance: Cross-Layer Load Balancing in Distributed MoE
  Inference" (arXiv 2608.07964v1), full text on the "Paper deep dive" page.
* [REVIEW] "EasyBalance：分布式 MoE 推理的跨层负载均衡", a review page that
  restates the equations and Algorithm 1 cleanly.
* [EP-ATLAS] "系统侧负载均衡：EPLB、LPLB、UltraEP 与 MoonEP", section 1
  (per-expert token counts T_e and per-rank load L_r), for the dispatch
  bookkeeping only.

Precision: floating point is float64 unless the step rounds to float32 by
definition (router gates are float32 outputs).  Integer work (selection,
counting sort, workloads, schedules) is exact.  Utilisation is an exact
``fractions.Fraction``.

Pinning status of every function is listed in each module's header.
"""
from .moe import (route, dispatch, swiglu_expert, expert_ffn, combine, widen,  # noqa: F401
                  gate_logits, rmsnorm)
from .balance import (group_workload, effective_workload, utilization, step_stats,  # noqa: F401
                      util_of, schedule, same_peak_windows, POLICIES)
from .engine import run_schedule_only, run_engine, moe_layer  # noqa: F401
