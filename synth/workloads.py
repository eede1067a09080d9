"""Model shapes and workloads (seeded, synthetic).

Each shape is a decoder-only GQA transformer; the work spec says how many
prompt tokens are prefilled, in which chunk size, and how many greedy decode
steps follow.  Values the workload descriptions leave unstated (RoPE base and
RMSNorm eps for some shapes, max_seq) take the readings recorded in the
design notes.
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Shape:
    name: str
    hidden: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    ffn_inter: int = 0
    n_experts: int = 0
    top_k: int = 0
    expert_inter: int = 0
    shared_inter: int = 0
    shared_gate: bool = False
    norm_topk_prob: int = 0
    tied: bool = False
    qkv_bias: bool = False
    rope_base: float = 10000.0
    rms_eps: float = 1e-5
    max_seq: int = 2048
    max_chunk: int = 128
    max_batch: int = 1
    kv_bf16: bool = False     # the oracle's KV cache stores bf16 values (workloads that fix a bf16 cache)
    sliding_window: int = 0   # 0: full causal attention; W > 0: the W most recent positions
    attn_softcap: float = 0.0  # 0: off; c > 0: scaled scores s -> c tanh(s / c)
    attn_sinks: bool = False  # one sink logit per query head and layer
    qk_norm: bool = False     # RMSNorm of every q and k head (gains q_norm, k_norm [d]) before RoPE
    weight_quant: int = 0     # 1: layer matrices and lm-head as int8 with a power-of-two scale per row
    kv_page_size: int = 0     # 0: contiguous KV per sequence; P: a pool of kv_pages pages of P positions
    kv_pages: int = 0

    @property
    def is_moe(self):
        return self.n_experts > 0

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_rows(self):
        return self.q_dim + 2 * self.kv_dim

    def with_(self, **kw):
        return replace(self, **kw)

    def layer_weight_bytes(self):
        """bf16 bytes of one layer's matrices (norm gains and biases excluded)."""
        H = self.hidden
        b = self.qkv_rows * H + H * self.q_dim
        if self.is_moe:
            b += self.n_experts * H + self.n_experts * 3 * self.expert_inter * H
            b += 3 * self.shared_inter * H + (H if self.shared_gate else 0)
        else:
            b += 3 * self.ffn_inter * H
        return 2 * b

    def n_params(self):
        p = self.n_layers * self.layer_weight_bytes() // 2 + self.vocab * self.hidden
        if not self.tied:
            p += self.vocab * self.hidden
        return p


@dataclass(frozen=True)
class Work:
    prompt: int
    chunk: int
    decode_steps: int
    batch: int = 1
    context: int = 0          # pre-filled synthetic KV length per sequence (batched long-context)


TINY = Shape("gqa-tiny-h256-l2", hidden=256, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=64,
             vocab=1024, ffn_inter=688, rope_base=1e4, max_seq=64, max_chunk=16)
C135M = Shape("gqa-135m-h576-l30", hidden=576, n_layers=30, n_heads=9, n_kv_heads=3, head_dim=64,
              vocab=49152, ffn_inter=1536, tied=True, rope_base=1e4, max_seq=2048)
C8B = Shape("gqa-8b-h4096-l32", hidden=4096, n_layers=32, n_heads=32, n_kv_heads=8, head_dim=128,
            vocab=128256, ffn_inter=14336, rope_base=5e5, max_seq=4096, max_chunk=512, kv_bf16=True)
MOE = Shape("moe-e60x1408-top4-h2048-l24", hidden=2048, n_layers=24, n_heads=16, n_kv_heads=16,
            head_dim=128, vocab=151936, n_experts=60, top_k=4, expert_inter=1408,
            shared_inter=5632, shared_gate=True, norm_topk_prob=0, qkv_bias=True,
            rope_base=1e4, max_seq=1024)
LONGCTX = C8B.with_(name="gqa-8b-h4096-l32-bs16-ctx32k", max_seq=32768 + 64, max_batch=16,
                    max_chunk=16)

WORKLOADS = {
    "tiny": (TINY, Work(prompt=16, chunk=16, decode_steps=16)),
    "135m": (C135M, Work(prompt=512, chunk=128, decode_steps=256)),
    "8b": (C8B, Work(prompt=2048, chunk=128, decode_steps=256)),
    "moe": (MOE, Work(prompt=512, chunk=128, decode_steps=128)),
    "longctx": (LONGCTX, Work(prompt=0, chunk=0, decode_steps=64, batch=16, context=32768)),
}
