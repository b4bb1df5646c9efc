"""The five synthetic workloads the path is measured and parity-tested on.

Shapes follow the 8B/13B-class models the iS-KV summary evaluates on
(page "iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental SVD",
sections "Summary" and "AIME Results"), and the LLaMA-2-13B MHA shape used in
"Tensor Decomposition of Transformer KV Caches", Table 3. Rows are synthetic:
X = G diag(s) W^T + 0.01 N with s_i = i^-alpha (see gen.py).

Two points the workload text leaves open are read plainly: the long-input
workload keeps the 128-row window of the other GQA workloads, and the
single-head workload draws its values with the same recipe as its keys.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    layers: int
    kv_heads: int
    q_heads: int
    head_dim: int
    block: int          # b: rows folded per update
    rank_k: int         # r_K
    rank_v: int         # r_V
    window: int         # w: exact recent rows kept at input precision
    decode_tokens: int  # tokens appended one at a time (each followed by a decode query)
    prefill_blocks: int  # blocks of b rows folded directly before decode
    alpha_k: float      # spectrum exponent of keys
    alpha_v: float      # spectrum exponent of values
    kv_dtype: str       # "f32" | "bf16": incoming rows, window, queries, outputs
    coord_dtype: str    # "f32" | "bf16": stored coordinates C = U Sigma
    noise: float = 0.01
    cfg_id: int = 0

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def units(self) -> int:
        """Independent (batch, layer, kv-head) units per K or per V."""
        return self.batch * self.layers * self.kv_heads

    @property
    def total_tokens(self) -> int:
        return self.prefill_blocks * self.block + self.decode_tokens

    @property
    def max_tokens(self) -> int:
        return self.total_tokens

    def final_counts(self):
        """(n, e, folds) after the whole run, following the window policy:
        prefill blocks fold straight into history; decode rows enter the
        window and the oldest b fold out once it holds w + b rows."""
        n = self.prefill_blocks * self.block
        folds = self.prefill_blocks
        e = 0
        for _ in range(self.decode_tokens):
            e += 1
            if e >= self.window + self.block:
                e -= self.block
                n += self.block
                folds += 1
        return n, e, folds


CONFIGS = [
    # Single head, single layer, fp32 end to end; keys and values both
    # spectrum exponent 1.2 (the workload names keys only; values reuse it).
    Workload("single_head_fp32", batch=1, layers=1, kv_heads=1, q_heads=1,
             head_dim=128, block=64, rank_k=32, rank_v=32, window=64,
             decode_tokens=1024, prefill_blocks=0, alpha_k=1.2, alpha_v=1.2,
             kv_dtype="f32", coord_dtype="f32", cfg_id=0),
    # Llama-3-8B-shaped GQA decode to 8192 tokens.
    Workload("llama3_8b_gqa_8k", batch=1, layers=32, kv_heads=8, q_heads=32,
             head_dim=128, block=64, rank_k=32, rank_v=32, window=128,
             decode_tokens=8192, prefill_blocks=0, alpha_k=1.5, alpha_v=0.8,
             kv_dtype="bf16", coord_dtype="bf16", cfg_id=1),
    # Qwen3-8B-shaped GQA decode to 32768 tokens, batch 4.
    Workload("qwen3_8b_gqa_32k", batch=4, layers=36, kv_heads=8, q_heads=32,
             head_dim=128, block=64, rank_k=24, rank_v=24, window=128,
             decode_tokens=32768, prefill_blocks=0, alpha_k=1.5, alpha_v=0.8,
             kv_dtype="bf16", coord_dtype="bf16", cfg_id=2),
    # Long input: 65536 prompt rows folded as 1024 blocks of 64, then 1024
    # decode tokens (window 128, as the other GQA workloads).
    Workload("long_input_64k", batch=1, layers=32, kv_heads=8, q_heads=32,
             head_dim=128, block=64, rank_k=32, rank_v=48, window=128,
             decode_tokens=1024, prefill_blocks=1024, alpha_k=1.5, alpha_v=0.8,
             kv_dtype="bf16", coord_dtype="bf16", cfg_id=3),
    # LLaMA-2-13B-shaped MHA stress, batch 16, 16384 tokens.
    Workload("llama2_13b_mha_16k", batch=16, layers=40, kv_heads=40, q_heads=40,
             head_dim=128, block=128, rank_k=64, rank_v=96, window=256,
             decode_tokens=16384, prefill_blocks=0, alpha_k=1.5, alpha_v=0.8,
             kv_dtype="bf16", coord_dtype="bf16", cfg_id=4),
]


def get_config(i_or_name) -> Workload:
    if isinstance(i_or_name, int):
        return CONFIGS[i_or_name]
    for c in CONFIGS:
        if c.name == i_or_name:
            return c
    raise KeyError(i_or_name)
