"""Seeded synthetic inputs for the KV-shared early-exit decoder.

This module only draws random numbers and names shapes; it holds none of the
method's arithmetic, so both the HIP path and the CPU oracle may consume what
it produces.

Model shapes are Llama-style decoders (the lead page, section "experiments",
names Llama3.2 1B with 16 layers and Llama3.1 8B with 32 layers); sizes below
are the standard published shapes of those model families, plus a tiny
decoder for fast checks.

Recipe:
  * weights: embedding and every linear ~ N(0, 0.02), drawn in fp32 from one
    ``torch.Generator`` seeded ``seed`` in the canonical order
    embed, then per layer q, k, v, o, gate, up, down, then lm_head (if untied),
    and rounded to bf16 (round-to-nearest-even, torch's cast);
  * RMSNorm gains are exactly 1.0;
  * tokens: uniform integers in [0, vocab) from a second generator seeded
    ``seed + 1``.

The generator lives on the device the tensors are made on, so the same seed
gives different (but reproducible) values on CPU and on GPU.  Whoever checks a
GPU result against the oracle hands both sides the very same tensors.
"""
from dataclasses import dataclass, asdict, replace

import torch


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    group_size: int
    tied_embeddings: bool
    rms_eps: float = 1e-5
    rope_theta: float = 500000.0

    def as_dict(self):
        return asdict(self)


TINY = ModelShape("tiny", 4, 256, 4, 2, 64, 1024, 1024, 64, False)
LLAMA_1B = ModelShape("llama-3.2-1b-shape", 16, 2048, 32, 8, 64, 8192, 128256, 128, True)
LLAMA_8B = ModelShape("llama-3.1-8b-shape", 32, 4096, 32, 8, 128, 14336, 128256, 128, False)

SHAPES = {"tiny": TINY, "1b": LLAMA_1B, "8b": LLAMA_8B}


@dataclass(frozen=True)
class Workload:
    """A decode workload: shape, batch, prompt length, decode steps, taus."""
    name: str
    shape: ModelShape
    batch: int
    prompt: int
    steps: int
    taus: tuple

    @property
    def max_seq(self):
        return self.prompt + self.steps


WORKLOADS = {
    "tiny": Workload("tiny-b2-t32", TINY, 2, 32, 16, (0.5,)),
    "1b": Workload("1b-b1-t256", LLAMA_1B, 1, 256, 256, (0.3, 0.5, 0.7)),
    "8b": Workload("8b-b1-t512", LLAMA_8B, 1, 512, 256, (0.5,)),
    "8b-b32": Workload("8b-b32-t1024", LLAMA_8B, 32, 1024, 512, (0.3, 0.5, 0.7, 0.9)),
    "8b-long": Workload("8b-b8-t16384", LLAMA_8B, 8, 16384, 128, (0.5,)),
}

LINEARS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def linear_shapes(shape: ModelShape):
    """(rows N, cols K) of each linear of one decoder layer, row-major [N][K]."""
    d, hd = shape.d_model, shape.head_dim
    return {
        "wq": (shape.n_q_heads * hd, d),
        "wk": (shape.n_kv_heads * hd, d),
        "wv": (shape.n_kv_heads * hd, d),
        "wo": (d, shape.n_q_heads * hd),
        "w_gate": (shape.ffn_dim, d),
        "w_up": (shape.ffn_dim, d),
        "w_down": (d, shape.ffn_dim),
    }


def _normal_bf16(gen, rows, cols, device):
    t = torch.empty((rows, cols), dtype=torch.float32, device=device)
    t.normal_(0.0, 0.02, generator=gen)
    return t.to(torch.bfloat16)


def make_weights(shape: ModelShape, seed: int = 0, device="cpu", n_layers=None):
    """Random-init weights of ``shape`` as bf16 tensors on ``device``.

    ``n_layers`` (default: all) truncates the decoder after that many layers
    while keeping the canonical draw order of the layers it keeps.
    """
    L = shape.n_layers if n_layers is None else n_layers
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    d = shape.d_model
    ones = torch.ones(d, dtype=torch.bfloat16, device=device)
    w = {"embed": _normal_bf16(gen, shape.vocab, d, device), "layers": []}
    for _ in range(L):
        lw = {"attn_norm": ones.clone(), "mlp_norm": ones.clone()}
        for name, (n, k) in linear_shapes(shape).items():
            lw[name] = _normal_bf16(gen, n, k, device)
        w["layers"].append(lw)
    w["final_norm"] = ones.clone()
    w["lm_head"] = None if shape.tied_embeddings else _normal_bf16(gen, shape.vocab, d, device)
    return w


def make_tokens(shape: ModelShape, batch: int, length: int, seed: int = 0):
    """Uniform token ids [batch, length] (int32, CPU) from a generator seeded seed+1."""
    gen = torch.Generator()
    gen.manual_seed(seed + 1)
    return torch.randint(0, shape.vocab, (batch, length), generator=gen, dtype=torch.int64).to(torch.int32)


def shrink(shape: ModelShape, **kw):
    """A copy of ``shape`` with some fields replaced (for small test decoders)."""
    return replace(shape, **kw)
