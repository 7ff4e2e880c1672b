"""The five synthetic workloads, shaped like the models the pages evaluate.

Shapes follow the pages' models: a tiny fp32 case, a GPT-2-small shape
(TIDE's convergence analysis lists GPT-2, 12 layers), a Llama-3.2-1B
decode step (River-LLM's smallest model), a Llama-3-8B shape for prefill
and decode (both pages' 8B models), and a long-context RidgeFill prefill
(d = 5120, 64 layers) at 32K and 64K tokens.

Layer numbering: blocks are 1..L and h^(0) is the embedding. A token that
exits after block e has h^(e); blocks e+1..L are skipped and filled.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    d: int
    L: int
    n_tokens: int                  # tokens in the evaluated batch
    dtype: str                     # "f32" or "bf16"
    route_layers: Tuple[int, ...]  # checkpoints e where the route runs
    b: int                         # router bottleneck (0: router off)
    n_kv_heads: int
    head_dim: int
    group: int                     # int4 group along the input dim
    sz_dtype: str                  # dtype of the int4 scale and zero
    n_slots: int                   # cache positions per layer
    use_maps: bool                 # ridge maps (True) or identity (False)
    n_calib: int = 0               # calibration tokens for the ridge fit
    ridge_lambda: float = 0.0
    tau: float = float("-inf")     # cosine threshold (A14 readings)
    theta: float = float("-inf")   # router threshold
    student_t: bool = False        # heavy-tailed states (long-context case)
    decode: bool = False           # tokens sit at random distinct slots
    slot_lo: int = 0               # decode slots are drawn from [slot_lo, n_slots)
    fill_lo: int = 0               # positional fill range [fill_lo, n - fill_tail)
    fill_tail: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def hd(self):
        return self.n_kv_heads * self.head_dim

    @property
    def n_maps(self):
        """Maps M_{e->l} for every route layer e and every l in e+1..L."""
        return sum(self.L - e for e in self.route_layers)


CONFIGS = {
    0: Config(idx=0, name="tiny-fp32", d=256, L=8, n_tokens=64, dtype="f32",
              route_layers=(2, 4, 6), b=32, n_kv_heads=2, head_dim=32,
              group=32, sz_dtype="f32", n_slots=128, use_maps=True,
              n_calib=512, ridge_lambda=1e-2, tau=0.9, theta=0.5),
    1: Config(idx=1, name="gpt2-small-prefill", d=768, L=12, n_tokens=4096,
              dtype="bf16", route_layers=(4,), b=128, n_kv_heads=12,
              head_dim=64, group=64, sz_dtype="bf16", n_slots=4096,
              use_maps=True, n_calib=2048, ridge_lambda=1e-2, tau=0.9,
              theta=0.5),
    2: Config(idx=2, name="llama3.2-1b-decode", d=2048, L=16, n_tokens=64,
              dtype="bf16", route_layers=tuple(range(8, 16)), b=0,
              n_kv_heads=8, head_dim=64, group=64, sz_dtype="bf16",
              n_slots=4096, use_maps=False, decode=True, slot_lo=1),
    3: Config(idx=3, name="llama3-8b-prefill", d=4096, L=32, n_tokens=8192,
              dtype="bf16", route_layers=tuple(range(3, 32, 4)), b=128,
              n_kv_heads=8, head_dim=128, group=128, sz_dtype="bf16",
              n_slots=8192, use_maps=True, n_calib=8192, ridge_lambda=1e-1,
              extra={"exit_early": 11, "exit_late": 31, "early_frac": 0.05}),
    4: Config(idx=4, name="ridgefill-long-prefill", d=5120, L=64,
              n_tokens=32768, dtype="bf16", route_layers=(16,), b=0,
              n_kv_heads=8, head_dim=128, group=128, sz_dtype="bf16",
              n_slots=32768, use_maps=True, n_calib=16384, ridge_lambda=1e-1,
              student_t=True, fill_lo=16, fill_tail=2048),
}

# decode variant of the 8B shape: 256 tokens at distinct slots in [0, 8192)
CONFIG_3D = Config(idx=3, name="llama3-8b-decode", d=4096, L=32, n_tokens=256,
                   dtype="bf16", route_layers=tuple(range(3, 32, 4)), b=128,
                   n_kv_heads=8, head_dim=128, group=128, sz_dtype="bf16",
                   n_slots=8192, use_maps=True, n_calib=8192, ridge_lambda=1e-1,
                   decode=True,
                   extra={"exit_early": 11, "exit_late": 31, "early_frac": 0.05})


def get_config(idx, **overrides) -> Config:
    from dataclasses import replace
    base = CONFIG_3D if idx == "3D" else CONFIGS[idx]
    return replace(base, **overrides) if overrides else base


def sigma(l: int) -> float:
    """Step size of the hidden-state random walk at block l (1-based)."""
    return 0.5 * 0.7 ** l
