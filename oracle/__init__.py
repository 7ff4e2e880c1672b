"""Reference oracle for the per-token exit-and-KV-fill step.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, float64 NumPy
statement of what the GPU library computes. It is imported by the tests,
by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``, and by nothing else. The product path never calls it and has
no CPU fallback: it shares no code, constant or helper with the HIP library.

Every function cites the passage of the source pages that defines the
operation. Sources (web pages, cited by title and section):

* River-LLM -- "River-LLM: Large Language Model Seamless Exit Based on KV
  Share" (Shen, Zou; paper summary page). Sections "前置知识" (state
  transition similarity), "核心方法", "方法步骤详情" (steps 1-4).
* TIDE -- "TIDE: Token-Informed Depth Execution for Per-Token Early Exit
  in LLM Inference" (reading notes). Sections "系统架构", "模块3: Post-Hoc
  Generation", "模块4: 融合 CUDA 内核", "关键公式" (formulas 3 and 4),
  "Figure 2".
* RidgeFill -- news article "RidgeFill: 免训练后层缓存填充". The method
  paragraph under "思路源头" and the closed-form ridge regression box.

Parity status of each function is stated in its docstring. Functions that
no test pins against something other than themselves say "parity
unpinned"; at present every exported function has at least one pin.
"""

from .river_oracle import (  # noqa: F401
    RULE_TOKEN,
    RULE_BATCH_MIN,
    route,
    compact,
    exit_projection,
    dequant_w4,
    kv_fill,
    kv_fill_rows,
    kv_fill_layer_rows,
    rope_half,
    ridge_fit,
    decode_step,
    router_labels,
    router_fit,
    exit_schedule_ops,
)
