"""The five synthetic workloads of the H2O decode path.

Each entry is the per-layer attention shape of a model family the H2O pages
evaluate on (OPT-6.7B, OPT-30B, GPT-NeoX-20B, LLaMA-7B; "Results and evidence"
of the Fanout summary "H2O: Heavy-Hitter Oracle for Efficient Generative
Inference") plus a fixed KV budget k = recent + heavy.  The 20% budget is the
operating point those pages report ("What to notice when reading").

No trained weights or dataset items are used: queries, keys and values are
seeded Gaussian draws with a planted skew direction (see ``synth.gen``), which
stand in for the models and the evaluation suites.

This module holds shapes and generator parameters only, none of the method's
arithmetic.
"""
from dataclasses import dataclass
import math


@dataclass(frozen=True)
class Workload:
    cid: int            # 1..5, part of every seed
    name: str
    batch: int
    heads: int
    head_dim: int
    prompt: int         # P
    steps: int          # T decode steps
    recent: int         # r, protected window (includes the token being decoded)
    heavy: int          # h, heavy-hitter slots
    kv_dtype: str       # "f32" or "bf16"
    skew: str           # "fraction" | "zipf" | "bursts" | "zipf_periodic"
    skew_frac: float = 0.0
    skew_amp: float = 3.0
    zipf_alpha: float = 0.0
    period: int = 0
    burst_len: int = 16
    query_amp: float = 1.5
    softmax_scale: float = 0.0  # 0: the default 1/sqrt(head_dim)

    @property
    def k(self) -> int:
        return self.recent + self.heavy

    @property
    def units(self) -> int:
        return self.batch * self.heads

    @property
    def n_positions(self) -> int:
        return self.prompt + self.steps

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.kv_dtype == "f32" else 2


WORKLOADS = {
    # Tiny single-layer trace, fp32: 8% of positions get a 3u key offset.
    "tiny_fp32": Workload(1, "tiny_fp32", 1, 2, 64, 64, 64, 16, 16, "f32",
                          "fraction", skew_frac=0.08),
    # OPT-6.7B-shaped layer, 20% of a 1024 length cap -> k = 204.
    "opt6.7b": Workload(2, "opt6.7b", 8, 32, 128, 512, 512, 102, 102, "bf16",
                        "fraction", skew_frac=0.05),
    # OPT-30B-shaped layer, 20% of 2048 -> k = 410; Zipf(1.1) key skew.
    "opt30b": Workload(3, "opt30b", 64, 56, 128, 1024, 1024, 205, 205, "bf16",
                       "zipf", zipf_alpha=1.1),
    # GPT-NeoX-20B-shaped layer, 20% of 6144 -> k = 1229, recent takes the odd slot.
    "neox20b": Workload(4, "neox20b", 16, 64, 96, 4096, 2048, 615, 614, "bf16",
                        "bursts", skew_frac=0.05),
    # LLaMA-7B-shaped long stream at a constant k = 256; Zipf(1.2) skew that
    # recurs with a period of 5000 positions.
    "llama7b_stream": Workload(5, "llama7b_stream", 1, 32, 128, 256, 200_000, 128, 128,
                               "bf16", "zipf_periodic", zipf_alpha=1.2, period=5000),
}

BY_ID = {w.cid: w for w in WORKLOADS.values()}

# The configuration the headline decode throughput is quoted on.
HEADLINE = "opt30b"
