"""Named workload shapes for hierarchical block-then-token sparse attention.

Each workload fixes the sizes of the four steps: the indexer vectors (width
``d_index``), the key block size ``block`` (B), the number of kept blocks
``top_m`` (m), the number of kept tokens ``top_k`` (k) and the attention heads.
Queries always sit at the last ``n_q`` positions of each sequence.

The block size of 128 and the block count of 64 follow the HISA page's
example values (section on the two-step method); the landmark mode with 4
landmark vectors per chunk follows the HiLS page (section 2.1, landmark
tokens), with a fixed random 0/1 projection standing in for the learned one.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_len: int
    n_q: int
    d_index: int
    block: int
    top_m: int
    top_k: int
    n_heads_q: int
    n_heads_kv: int
    head_dim: int = 128
    n_landmarks: int = 1
    needles: int = 0
    # > 0: decode over sequences of different lengths, uniform in
    # [varlen_min, seq_len] (seq_len is then the cache capacity; n_q == 1)
    varlen_min: int = 0
    # > 0: three-level selection, super-blocks of `group` blocks of which
    # `top_m2` are kept before the blocks are chosen among theirs
    group: int = 0
    top_m2: int = 0
    # True: every query head selects its own chunks from Q against
    # landmarks of K (no indexer vectors, no token top-k)
    per_head: bool = False
    seed: int = 0
    description: str = ""

    @property
    def scale(self) -> float:
        # softmax temperature 1/sqrt(head_dim), rounded to fp32 once so that
        # every consumer uses the same value
        import numpy as np
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def n_blocks(self) -> int:
        return (self.seq_len + self.block - 1) // self.block

    @property
    def n_super(self) -> int:
        return (self.n_blocks + self.group - 1) // self.group if self.group else 0

    def query_pos(self, i: int) -> int:
        """Absolute position of query i (queries are the last n_q tokens)."""
        return self.seq_len - self.n_q + i

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_prefill_4k": Workload(
        name="tiny_prefill_4k", batch=1, seq_len=4096, n_q=4096, d_index=64,
        block=64, top_m=8, top_k=256, n_heads_q=1, n_heads_kv=1,
        description="causal prefill, L=4096, B=64, m=8, k=256, 1 head"),
    "prefill_64k": Workload(
        name="prefill_64k", batch=1, seq_len=65536, n_q=65536, d_index=128,
        block=128, top_m=64, top_k=2048, n_heads_q=16, n_heads_kv=1,
        description="causal prefill, L=65536, B=128, m=64, k=2048, 16:1 GQA"),
    "decode_128k": Workload(
        name="decode_128k", batch=32, seq_len=131072, n_q=1, d_index=128,
        block=128, top_m=64, top_k=2048, n_heads_q=16, n_heads_kv=1, needles=4,
        description="decode, batch 32, L=131072, 4 planted needle blocks"),
    "chunked_prefill_512k": Workload(
        name="chunked_prefill_512k", batch=1, seq_len=524288, n_q=4096,
        d_index=128, block=128, top_m=128, top_k=4096, n_heads_q=32, n_heads_kv=2,
        description="4096 new queries against a 524288-token causal context"),
    "decode_512k": Workload(
        name="decode_512k", batch=4, seq_len=524288, n_q=1, d_index=128,
        block=128, top_m=128, top_k=4096, n_heads_q=32, n_heads_kv=2,
        description="decode, batch 4, L=524288"),
    "decode_varlen_128k": Workload(
        name="decode_varlen_128k", batch=32, seq_len=131072, n_q=1, d_index=128,
        block=128, top_m=64, top_k=2048, n_heads_q=16, n_heads_kv=1, varlen_min=65536,
        description="decode, batch 32, cache capacity 131072, lengths uniform in [65536, 131072]"),
    "decode_3level_1m": Workload(
        name="decode_3level_1m", batch=8, seq_len=1048576, n_q=1, d_index=128,
        block=128, top_m=64, top_k=2048, n_heads_q=16, n_heads_kv=1, needles=4,
        group=16, top_m2=32,
        description="decode, batch 8, L=1048576, super-blocks of 16 blocks, 32 kept, then 64 blocks"),
    "head_decode_512k": Workload(
        name="head_decode_512k", batch=4, seq_len=524288, n_q=1, d_index=128,
        block=64, top_m=32, top_k=32 * 64, n_heads_q=32, n_heads_kv=4, n_landmarks=4,
        per_head=True, needles=1,
        description="per-head chunk selection from Q (HiLS-style), decode, batch 4, L=524288, "
                    "chunks of 64 with 4 landmarks, 32 kept per head, 32 query heads / 4 kv heads"),
    "landmark_decode_1m": Workload(
        name="landmark_decode_1m", batch=2, seq_len=1048576, n_q=1, d_index=128,
        block=128, top_m=256, top_k=256 * 128, n_heads_q=16, n_heads_kv=1,
        n_landmarks=4,
        description="chunk-landmark decode, batch 2, L=1048576, 4 landmarks/block"),
}
