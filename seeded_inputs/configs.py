"""Model shapes and seeds of the five synthetic workloads.

Shapes follow the workload list of the block-verification study (a tiny 2-layer
decoder, a Qwen3-0.6B-shaped and a Qwen3-8B-shaped bf16 target, a Gemma-style
int4 target, and an 8B-shaped long-context stress case).  Model details the
workloads leave open are fixed here as plain readings: norm gains 1.0, no
biases, no QK-norm, rotate-half RoPE with theta 1e4 for every model, GQA head j
reads KV head j // (n_q / n_kv), attention scale 1/sqrt(head_dim), and the LM
head tied to the embedding.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    act: str = "swiglu"          # "swiglu" (SiLU gate) or "geglu" (tanh-GELU gate)
    weight_fmt: str = "bf16"     # linears: "bf16" or "int4" (symmetric, group 64, bf16 scales)
    rms_eps: float = 1e-6
    rope_theta: float = 1e4
    tied: bool = True            # LM head is the embedding table
    page_size: int = 16
    max_ctx: int = 2048          # KV capacity in positions
    max_k: int = 16              # most draft tokens per verify (rows = k + 1)
    seed: int = 1
    gain_std: float = 0.0        # 0 -> all norm gains exactly 1.0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_dim(self) -> int:
        return self.q_dim + 2 * self.kv_dim

    def linear_shapes(self):
        """Canonical [out, in] shapes of one layer's linears, in generation order."""
        d, f = self.d_model, self.d_ff
        return {
            "wq": (self.q_dim, d),
            "wk": (self.kv_dim, d),
            "wv": (self.kv_dim, d),
            "wo": (d, self.q_dim),
            "wg": (f, d),
            "wu": (f, d),
            "wd": (d, f),
        }

    def weight_bytes_per_forward(self) -> int:
        """Bytes of weights one forward streams (linears, tied LM head, gains)."""
        lin = 0
        for (o, i) in self.linear_shapes().values():
            if self.weight_fmt == "int4":
                lin += o * i // 2 + o * (i // 64) * 2
            else:
                lin += o * i * 2
        gains = (2 * self.d_model) * self.n_layers + self.d_model
        return lin * self.n_layers + self.vocab * self.d_model * 2 + gains * 2

    def kv_bytes_per_token(self) -> int:
        return self.n_layers * 2 * self.n_kv_heads * self.head_dim * 2


PRESETS = {
    "tiny": ModelConfig("tiny", 2, 256, 4, 2, 64, 1024, 2048,
                        max_ctx=256, max_k=8, seed=1),
    "q06b": ModelConfig("q06b", 28, 1024, 16, 8, 128, 3072, 151936,
                        max_ctx=1024, max_k=8, seed=2),
    "gemma_int4": ModelConfig("gemma_int4", 35, 1536, 12, 2, 128, 6144, 262144,
                              act="geglu", weight_fmt="int4",
                              max_ctx=256, max_k=16, seed=3),
    "q8b": ModelConfig("q8b", 36, 4096, 32, 8, 128, 12288, 151936,
                       max_ctx=2048, max_k=16, seed=4),
    "q8b_stress": ModelConfig("q8b_stress", 36, 4096, 32, 8, 128, 12288, 151936,
                              max_ctx=32768, max_k=32, seed=4),
}


def get_config(name: str, **overrides) -> ModelConfig:
    cfg = PRESETS[name]
    return replace(cfg, **overrides) if overrides else cfg


def layer_variant(name: str, n_layers: int = 2, vocab: int = 512, **overrides) -> ModelConfig:
    """A preset's layer shape with fewer layers and a cut vocabulary (for CPU pins)."""
    cfg = PRESETS[name]
    return replace(cfg, name=f"{cfg.name}_L{n_layers}_V{vocab}", n_layers=n_layers,
                   vocab=vocab, **overrides)
