"""The five synthetic workloads the layer is checked and measured on.

Shapes follow the Mamba-2 layers of the models the pages describe:
head_dim 64, d_state 128, conv kernel 4, expand 2, n_groups 8, chunk 128
("Nemotron-H style Hybrid Mamba-Transformer 3B feasibility study",
tables 1.4 and 1.5 and section 2.2).  Nothing here computes any part of the
layer; it only names sizes.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int            # prefill tokens per sequence (decode: 1)
    nheads: int
    headdim: int = 64
    dstate: int = 128
    ngroups: int = 8
    chunk: int = 128
    width: int = 4          # conv kernel
    dtype: str = "bf16"     # activations: "f32" or "bf16"; params/state fp32
    initial_state: bool = False
    decode_steps: int = 0   # > 0: a chain of one-token decode steps
    seed: int = 8000
    expand: int = 2         # d_inner / d_model of the block around the layer

    @property
    def d_inner(self) -> int:
        return self.nheads * self.headdim

    @property
    def d_model(self) -> int:
        return self.d_inner // self.expand

    @property
    def d_in_proj(self) -> int:
        """in_proj outputs: z | x | B | C | dt."""
        return 2 * self.d_inner + 2 * self.ngroups * self.dstate + self.nheads

    @property
    def cdim(self) -> int:
        return self.d_inner + 2 * self.ngroups * self.dstate

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny fp32 prefill: the case the oracle finishes in well under a second
    "tiny_f32_b1_l512_h4": Workload("tiny_f32_b1_l512_h4", batch=1, seqlen=512, nheads=4,
                                    ngroups=1, dtype="f32", seed=8000),
    # Nemotron-H-8B Mamba-2 layer: d_model 4096, expand 2 -> 128 heads x 64
    "nemotron_h_8b_b4_l8192": Workload("nemotron_h_8b_b4_l8192", batch=4, seqlen=8192,
                                       nheads=128, seed=8001),
    # Nemotron-3-Nano layer: 64 heads x 64, with a nonzero initial state
    "nemotron3_nano_b8_l4096": Workload("nemotron3_nano_b8_l4096", batch=8, seqlen=4096,
                                        nheads=64, initial_state=True, seed=8002),
    # long context, one sequence of 131072 tokens, 80 heads (d_model 2560, expand 2)
    "long_ctx_3b_b1_l131072": Workload("long_ctx_3b_b1_l131072", batch=1, seqlen=131072,
                                       nheads=80, seed=8003),
    # decode: 256 sequences, 1000 chained one-token steps, fp32 state
    "decode_b256_h128_x1000": Workload("decode_b256_h128_x1000", batch=256, seqlen=1,
                                       nheads=128, initial_state=True, decode_steps=1000,
                                       seed=8004),
}

ORDER = list(WORKLOADS)
PREFILL_MAIN = "nemotron_h_8b_b4_l8192"
DECODE_MAIN = "decode_b256_h128_x1000"
