"""Workload table for gated SDPA (G1 gate on the SDPA output).

Shapes follow the pages' setting: context 4096 for pre-training and 32k for the
long-context extension ("2025_GatedAttention", §1.3.1 and §1.4.4), GQA attention
(§1.3.1), and KV-cache decode (§1.3.1, GQA explainer).  All draws are N(0, 1)
except the gate weight W_theta, drawn N(0, 1/d_model) (the second parameter is
the variance), so gate logits are roughly N(0, 1).
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    S: int            # query length (1 for decode)
    d_model: int
    Hq: int
    Hkv: int
    D: int
    mode: str         # "elementwise" | "headwise" | "none"
    dtype: str        # "fp32" | "bf16"
    L: int = 0        # KV-cache length for decode (0 for prefill: keys = queries)
    sink_scale: float = 1.0   # factor applied to the keys of token 0 (power of two => exact)
    description: str = ""

    @property
    def decode(self) -> bool:
        return self.L > 0

    @property
    def Skv(self) -> int:
        return self.L if self.decode else self.S

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def N(self) -> int:
        """Gate width: one column per (head, dim) for elementwise, one per head for headwise."""
        if self.mode == "elementwise":
            return self.Hq * self.D
        if self.mode == "headwise":
            return self.Hq
        return 0

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)

    # Algorithmic work, counted the method's way: causal pairs j <= i (with the
    # queries aligned to the end of the key range) x 4*D flops, plus 2*M*d_model*N
    # for the gate projection.
    def causal_pairs(self) -> int:
        off = self.Skv - self.S
        # sum over i in [0, S) of (i + off + 1)
        return self.S * (self.S + 1) // 2 + self.S * off

    def attention_flops(self) -> int:
        return 4 * self.D * self.B * self.Hq * self.causal_pairs()

    def gate_flops(self) -> int:
        return 2 * self.B * self.S * self.d_model * self.N

    def total_flops(self) -> int:
        return self.attention_flops() + self.gate_flops()

    # Backward, counted the same way: the four products the gradients need
    # (dP = dY·Vᵀ, dV = Pᵀ·dY, dQ = dS·K, dK = dSᵀ·Q: 8*D flops per causal pair;
    # recomputing S = Q·Kᵀ is not counted) plus the gate branch's two products
    # (dX = dZ·W_θᵀ and dW_θ = Xᵀ·dZ, 2*M*d_model*N flops each).
    def backward_attention_flops(self) -> int:
        return 8 * self.D * self.B * self.Hq * self.causal_pairs()

    def backward_flops(self) -> int:
        return self.backward_attention_flops() + 2 * self.gate_flops()

    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def decode_bytes(self) -> dict:
        """Bytes a decode step must move at least once: inputs read once, output written once."""
        e = self.elem_bytes()
        kv = 2 * self.B * self.L * self.Hkv * self.D * e
        w = self.d_model * self.N * e
        x = self.B * self.d_model * e
        q = self.B * self.Hq * self.D * e
        y = self.B * self.Hq * self.D * e
        return {"kv": kv, "w": w, "x": x, "q": q, "y": y, "total": kv + w + x + q + y}


CONFIGS = {
    c.name: c for c in [
        Config("tiny_fp32", B=1, S=128, d_model=256, Hq=4, Hkv=4, D=64,
               mode="elementwise", dtype="fp32",
               description="tiny fp32 MHA, elementwise gate, W 256x256"),
        Config("dense_prefill", B=2, S=4096, d_model=2048, Hq=16, Hkv=16, D=128,
               mode="elementwise", dtype="bf16",
               description="bf16 dense-model-like prefill, elementwise gate, W 2048x2048"),
        Config("gqa_prefill", B=1, S=8192, d_model=4096, Hq=32, Hkv=4, D=128,
               mode="headwise", dtype="bf16",
               description="bf16 GQA (group 8) prefill, headwise gate, W 4096x32"),
        Config("long_prefill", B=1, S=32768, d_model=2048, Hq=16, Hkv=2, D=128,
               mode="elementwise", dtype="bf16", sink_scale=8.0,
               description="bf16 32k prefill, GQA group 8, elementwise gate, token-0 keys x8"),
        Config("decode", B=64, S=1, d_model=4096, Hq=32, Hkv=8, D=128, L=16384,
               mode="elementwise", dtype="bf16",
               description="bf16 decode: 1 query token vs a 16384-long KV cache, GQA group 4"),
    ]
}


def get_config(name: str) -> Config:
    return CONFIGS[name]
