"""The five synthetic workloads the verify step is tested and measured on.

Shapes follow the model pairs and serving conditions the pages discuss:
a tiny case the oracle finishes in seconds, a Qwen3-1.7B/0.6B-shaped pair at
batch 1, a low-concurrency sweep, a Llama-3-8B-shaped serving batch of 64
(the headline workload) and a Llama-3-70B-shaped single-GPU share at batch
256.  Logits are N(0, 2) (standard deviation 2; the tiny case N(0, 1)) and
the draft is the target plus N(0, sigma) noise.

``SIGMA_FOR_ALPHA`` maps a target per-token acceptance alpha (at T = 1, for
N(0, 2) logits over a large vocabulary) to the draft noise sigma that gives
it; the CPU tests re-measure alpha with the oracle for these values.
"""

from dataclasses import dataclass, field
from typing import Tuple

__all__ = ["Workload", "CONFIGS", "get_config", "SIGMA_FOR_ALPHA"]

SIGMA_FOR_ALPHA = {0.5: 1.35, 0.6: 1.05, 0.7: 0.77, 0.8: 0.51, 0.9: 0.25}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    V: int
    logit_dtype: str
    logit_std: float
    draft_sigma: float
    temperatures: Tuple[float, ...]
    Hq: int
    Hkv: int
    D: int
    ctx: Tuple[int, int]
    attn_dtype: str
    notes: str = ""
    sweep: dict = field(default_factory=dict, compare=False, hash=False)


CONFIGS = {
    "tiny": Workload(
        name="tiny", B=1, K=4, V=32, logit_dtype="f32", logit_std=1.0,
        draft_sigma=0.5, temperatures=(1.0, 0.0), Hq=1, Hkv=1, D=64,
        ctx=(128, 128), attn_dtype="f32",
        notes="1e5 trials batched along B at T=1 plus a greedy pass"),
    "qwen_b1": Workload(
        name="qwen_b1", B=1, K=8, V=151936, logit_dtype="bf16", logit_std=2.0,
        draft_sigma=0.51, temperatures=(0.0, 1.0), Hq=16, Hkv=8, D=128,
        ctx=(2048, 2048), attn_dtype="bf16",
        sweep={"K": (2, 4, 6, 8), "alpha": (0.5, 0.6, 0.7, 0.8, 0.9)}),
    "lowconc": Workload(
        name="lowconc", B=8, K=7, V=151936, logit_dtype="bf16", logit_std=2.0,
        draft_sigma=0.51, temperatures=(0.0, 0.6, 1.0, 1.2), Hq=16, Hkv=8,
        D=128, ctx=(1024, 4096), attn_dtype="bf16",
        sweep={"B": (1, 2, 4, 8)}),
    "llama8b_b64": Workload(
        name="llama8b_b64", B=64, K=7, V=128256, logit_dtype="bf16",
        logit_std=2.0, draft_sigma=0.51, temperatures=(1.0, 0.0), Hq=32,
        Hkv=8, D=128, ctx=(2048, 8192), attn_dtype="bf16",
        notes="headline workload: T=1, alpha ~ 0.8"),
    "llama70b_b256": Workload(
        name="llama70b_b256", B=256, K=7, V=128256, logit_dtype="bf16",
        logit_std=2.0, draft_sigma=0.51, temperatures=(0.0, 1.0), Hq=64,
        Hkv=8, D=128, ctx=(8192, 32768), attn_dtype="bf16",
        sweep={"alpha": (0.6, 0.8, 0.9)}),
}


def get_config(name):
    return CONFIGS[name]
