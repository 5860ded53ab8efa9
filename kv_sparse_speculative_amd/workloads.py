"""The five synthetic per-layer workloads the library is checked and measured on.

Shapes follow the models and settings of MagicDec's evaluation (Llama-3.1-8B layers at
8k-100k prefill, Section 5 and Tables 2, 4 and 6; Qwen-2.5-32B at 32k, Table 7); the data are
seeded synthetic tensors, not the paper's datasets.
"""

from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16": the stored KV / query type
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    prompt: Tuple[int, int]         # prompt length range, inclusive (lo == hi: homogeneous)
    gamma: int                      # speculation length; verify runs gamma + 1 queries
    streaming: Optional[Tuple[int, int]]     # (sink, window) StreamingLLM draft set
    snapkv: Optional[Tuple[int, int, int]]   # (budget, observation window, pool kernel)
    vocab: int
    block_size: int = 16
    shuffled_blocks: bool = False   # shuffled block table (else identity)
    planted_frac: float = 0.0       # share of candidate keys planted near window queries
    seed: int = 0

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def ragged(self):
        return self.prompt[0] != self.prompt[1]


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", "f32", 2, 8, 2, 64, (512, 512), 3, (4, 60), (64, 16, 7), 64,
                 seed=1001),
        Workload("llama8b_ctx8k", "bf16", 32, 32, 8, 128, (8192, 8192), 3, None, (512, 32, 7),
                 128256, planted_frac=0.02, seed=1002),
        Workload("llama8b_ctx32k", "bf16", 64, 32, 8, 128, (32000, 32000), 4, (16, 496),
                 (512, 32, 7), 128256, planted_frac=0.02, seed=1003),
        Workload("llama8b_ctx100k", "bf16", 16, 32, 8, 128, (100000, 100000), 4, None,
                 (1024, 64, 7), 128256, planted_frac=0.02, seed=1004),
        Workload("qwen32b_ragged", "bf16", 128, 40, 8, 128, (4096, 16384), 3, None,
                 (2048, 32, 7), 152064, shuffled_blocks=True, planted_frac=0.02, seed=1005),
    ]
}

# The measured workload: Llama-3.1-8B-shaped layer, batch 64, 32000-token context.
HEADLINE = "llama8b_ctx32k"
