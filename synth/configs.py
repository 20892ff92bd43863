"""The five layer workloads, named by their shapes.

Shapes and distributions follow the ZONOS2 backbone description (Zyphra,
"ZONOS2 Technical Report" digest, architecture item 5: 16 experts per MoE
layer, top-1 routing, top-2 in the last MoE layer; item 6: a per-expert bias
vector b_l).  The model width d_model=2048 and expert width d_ff=3072 are
assumed shapes: the pages give only 8B total / 900M active parameters.

Distribution notation N(0, v) is read with v as the variance everywhere.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class LayerConfig:
    cid: int
    name: str
    T: int            # tokens in the batch
    d: int            # d_model
    E: int            # experts
    F: int            # d_ff of each SwiGLU expert
    k: int            # experts per token
    dtype: str        # "f32" or "bf16": storage of activations and weights
    bias: str         # "normal" | "zero" | "zipf"
    eps: float = 1e-6
    # Weights of configs with the same family are the same tensors.
    family: str = field(default="")

    @property
    def assignments(self) -> int:
        return self.T * self.k


WORKLOADS = {
    0: LayerConfig(0, "tiny_fp32_T64_d256_E4_F512_top1", T=64, d=256, E=4, F=512, k=1,
                   dtype="f32", bias="normal", family="d256_E4_F512"),
    1: LayerConfig(1, "decode_bf16_T32_d2048_E16_F3072_top1", T=32, d=2048, E=16, F=3072,
                   k=1, dtype="bf16", bias="normal", family="d2048_E16_F3072"),
    2: LayerConfig(2, "prefill_bf16_T4096_d2048_E16_F3072_top1_b0", T=4096, d=2048, E=16,
                   F=3072, k=1, dtype="bf16", bias="zero", family="d2048_E16_F3072"),
    3: LayerConfig(3, "top2_bf16_T4096_d2048_E16_F3072", T=4096, d=2048, E=16, F=3072, k=2,
                   dtype="bf16", bias="normal", family="d2048_E16_F3072"),
    4: LayerConfig(4, "skewed_bf16_T16384_d2048_E16_F3072_top1_zipf", T=16384, d=2048, E=16,
                   F=3072, k=1, dtype="bf16", bias="zipf", family="d2048_E16_F3072"),
}

# Zipf exponent and rank count for the skewed workload.  Zipf(1.2) over 15
# ranks puts 37% of tokens on the hottest expert; the 16th expert is held
# empty so that at least one expert receives no tokens.
ZIPF_S = 1.2
ZIPF_RANKS = 15
ZIPF_EMPTY_BIAS = -1.0e4


def get_config(cid: int) -> LayerConfig:
    return WORKLOADS[int(cid)]
