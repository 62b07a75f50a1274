"""Model shapes and workloads of the decode benchmarks (plain data, no arithmetic).

Every workload is a Llama-style decoder with random-init bf16 weights; the
shapes are those of the public model families they are named after.  The
39-token prompt / 512 greedy tokens workload is the one the MPK write-up
measures on ("Compilar LLM en un MegaKernel ...", section "Valor central de
MPK"); its prompt text is not given, so random ids stand in for it.
"""
from dataclasses import dataclass, replace, asdict


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 500000.0
    tie_embeddings: bool = False


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    batch: int
    prompt_len: int
    decode_steps: int
    prompt_seed: int
    weight_seed: int = 0

    @property
    def max_seq(self) -> int:
        return self.prompt_len + self.decode_steps


TINY = ModelShape("tiny", 2, 256, 4, 2, 64, 688, 1024, 1e-5, 10000.0, False)
LLAMA1B = ModelShape("llama1b", 16, 2048, 32, 8, 64, 8192, 128256, 1e-5, 500000.0, True)
LLAMA8B = ModelShape("llama8b", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, False)
LLAMA70B = ModelShape("llama70b", 80, 8192, 64, 8, 128, 28672, 128256, 1e-5, 500000.0, False)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, 1, 8, 16, 1000),
    "llama1b": Workload("llama1b", LLAMA1B, 1, 39, 512, 1001),
    "llama8b": Workload("llama8b", LLAMA8B, 1, 39, 512, 1002),
    "llama8b_b8_kv4096": Workload("llama8b_b8_kv4096", LLAMA8B, 8, 4096, 128, 1003),
    "llama70b_b64": Workload("llama70b_b64", LLAMA70B, 64, 512, 64, 1004),
}


def with_layers(shape: ModelShape, n_layers: int) -> ModelShape:
    """The same shape with fewer layers (for tests that need full-width layers fast)."""
    return replace(shape, name=f"{shape.name}_L{n_layers}", n_layers=n_layers)


def shape_dict(shape: ModelShape) -> dict:
    return asdict(shape)


# --- tensor ids of the counter-based generator --------------------------------
# Every tensor draws from its own stream, keyed by (seed, tensor id).
TID_EMBED = 0
TID_LM_HEAD = 1
TID_FINAL_NORM = 2
TID_PROMPT = 3
LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


def layer_tid(layer: int, name: str) -> int:
    return 16 + 16 * layer + LAYER_TENSORS.index(name)


def weight_shapes(shape: ModelShape) -> dict:
    """name -> (rows, cols) of every weight; matrices are [out, in] row-major."""
    H, F, V = shape.hidden, shape.ffn, shape.vocab
    qd = shape.n_q_heads * shape.head_dim
    kd = shape.n_kv_heads * shape.head_dim
    out = {"embed": (V, H), "final_norm": (1, H)}
    if not shape.tie_embeddings:
        out["lm_head"] = (V, H)
    for l in range(shape.n_layers):
        out[f"layers.{l}.attn_norm"] = (1, H)
        out[f"layers.{l}.wq"] = (qd, H)
        out[f"layers.{l}.wk"] = (kd, H)
        out[f"layers.{l}.wv"] = (kd, H)
        out[f"layers.{l}.wo"] = (H, qd)
        out[f"layers.{l}.ffn_norm"] = (1, H)
        out[f"layers.{l}.w_gate"] = (F, H)
        out[f"layers.{l}.w_up"] = (F, H)
        out[f"layers.{l}.w_down"] = (H, F)
    return out


def tensor_id(name: str) -> int:
    if name == "embed":
        return TID_EMBED
    if name == "lm_head":
        return TID_LM_HEAD
    if name == "final_norm":
        return TID_FINAL_NORM
    _, l, t = name.split(".")
    return layer_tid(int(l), t)
