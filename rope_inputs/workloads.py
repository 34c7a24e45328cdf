"""The five synthetic workloads (shapes, seeds, id structure).

Sizes and structure follow the workloads the rotary-embedding pages imply:
an fp32 toy case with a per-token (B, S, R/2) cache, an fp16 prefill with a
gathered (M, R/2) cache, an fp32 partial interleaved rotation, a multimodal
M-RoPE prefill with text spans and image-patch grids, and an fp16 decode step
rotating Q and K together. Random values come only from rope_inputs.generators;
the cos/sin tables are NOT built here (that is the method's arithmetic): each
workload names the table it needs by (rows, base, rotary_dim, scaling) and the
caller builds it with its own implementation.

Seeds: 0x5EED0000 + 16 * index + tensor, tensor 0 = X (or Q), 1 = ids,
2 = K, 3 = out-of-range id selection.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

from .generators import SplitMix64, normal_tensor, sample_without_replacement, uniform_ints


def seed(index: int, tensor: int) -> int:
    return 0x5EED0000 + 16 * index + tensor


@dataclass
class Workload:
    index: int
    name: str
    op: str                      # "rope", "mrope", "rope_qk", "qkv_packed", "kv_append", "qk_norm"
    dtype: type
    x_shape: Tuple[int, ...]     # X, or Q for rope_qk
    num_heads: int = 0
    rotary_embedding_dim: int = 0
    interleaved: int = 0
    has_ids: bool = True
    cache_rows: int = 0          # M of the (M, R/2) table; for no-ids the positions 0..S-1
    cache_base: float = 10000.0
    scaling: float = 1.0
    k_shape: Optional[Tuple[int, ...]] = None
    kv_num_heads: int = 0
    mrope_section: Optional[Tuple[int, int, int]] = None
    mrope_layout: int = 0
    scale: float = 1.0
    description: str = ""
    extra: dict = field(default_factory=dict)

    # -- derived sizes -----------------------------------------------------
    @property
    def rank(self) -> int:
        return len(self.x_shape)

    @property
    def head_size(self) -> int:
        if self.rank == 4:
            return self.x_shape[3]
        if self.op == "qkv_packed":
            return self.x_shape[2] // (self.num_heads + 2 * self.kv_num_heads)
        return self.x_shape[2] // self.num_heads

    @property
    def rotary_dim(self) -> int:
        return self.rotary_embedding_dim or self.head_size

    @property
    def half(self) -> int:
        return self.rotary_dim // 2

    @property
    def batch(self) -> int:
        return self.x_shape[0]

    @property
    def seq(self) -> int:
        return self.x_shape[2] if self.rank == 4 else self.x_shape[1]

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def heads(self) -> int:
        return self.x_shape[1] if self.rank == 4 else self.num_heads

    @property
    def itemsize(self) -> int:
        return np.dtype(self.dtype).itemsize

    def algorithmic_bytes(self, onthefly: bool = False) -> int:
        """X read + Y write + one coefficient row (cos and sin) per token + ids.

        On the fly the coefficient term is the inv_freq vector (4 bytes per
        slot) read once instead of per-token table rows."""
        xy = 2 * int(np.prod(self.x_shape)) * self.itemsize
        if self.k_shape is not None:
            xy += 2 * int(np.prod(self.k_shape)) * self.itemsize
        if self.op in ("kv_append", "kv_append_norm"):
            # Q read + written, K and V read and written to one cache row each,
            # the per-sequence lengths (int32) instead of ids
            xy += 2 * int(np.prod(self.k_shape)) * self.itemsize
            w = 2 * self.head_size * self.itemsize if self.op == "kv_append_norm" else 0
            return xy + self.tokens * 2 * self.half * self.itemsize + self.batch * 4 + w
        coef = 4 * self.half if onthefly else self.tokens * 2 * self.half * self.itemsize
        n_id_streams = 3 if self.op == "mrope" else (1 if self.has_ids else 0)
        weights = 2 * self.head_size * self.itemsize if self.op in ("qk_norm", "kv_append_norm") else 0
        return xy + coef + n_id_streams * self.tokens * 8 + weights

    def tokens_heads(self) -> int:
        """(token, head) rows rotated."""
        th = self.tokens * self.heads
        if self.k_shape is not None or self.op == "qkv_packed":
            th += self.tokens * self.kv_num_heads
        return th

    # -- inputs ------------------------------------------------------------
    def make_x(self) -> np.ndarray:
        return normal_tensor(seed(self.index, 0), self.x_shape, self.dtype)

    def make_k(self) -> np.ndarray:
        return normal_tensor(seed(self.index, 2), self.k_shape, self.dtype)

    def make_norm_weights(self):
        """qk_norm: (q_weight, k_weight), values 1 + N(0, 1/16) rounded to the type."""
        out = []
        for t in (5, 6):
            v = 1.0 + 0.25 * normal_tensor(seed(self.index, t), (self.head_size,), np.float32)
            out.append(normal_like_type(v, self.dtype))
        return tuple(out)

    def make_v(self) -> np.ndarray:
        return normal_tensor(seed(self.index, 4), self.k_shape, self.dtype)

    def make_lengths(self) -> np.ndarray:
        """kv_append: per-sequence total key lengths U[1, cache_seq] (int32);
        a prompt: every sequence holds its S new tokens only."""
        if self.extra.get("prompt"):
            return np.full((self.batch,), self.seq, np.int32)
        cap = self.extra["cache_seq"]
        return (uniform_ints(seed(self.index, 1), (self.batch,), cap) + 1).astype(np.int32)

    def make_ids(self) -> Optional[np.ndarray]:
        if self.op == "mrope" and self.extra.get("ids") == "decode":
            # a text token after the prompt: the three streams share its position
            p = uniform_ints(seed(self.index, 1), (self.batch, self.seq), self.cache_rows)
            return np.stack([p, p, p])
        if self.op == "mrope":
            return mrope_ids(self.index, self.batch, self.seq, self.cache_rows,
                             self.extra.get("oob_fraction", 0.01))
        if not self.has_ids:
            return None
        kind = self.extra.get("ids", "uniform")
        if kind == "offset_arange":
            off = uniform_ints(seed(self.index, 1), (self.batch, 1), self.extra["offset_bound"])
            return off + np.arange(self.seq, dtype=np.int64)[None, :]
        return uniform_ints(seed(self.index, 1), (self.batch, self.seq), self.extra["id_bound"])

    def cache_positions(self) -> np.ndarray:
        """Rows the table is built for: 0..M-1 (gathered) or 0..S-1 per batch."""
        if self.has_ids or self.op == "mrope":
            return np.arange(self.cache_rows, dtype=np.int64)
        return np.arange(self.seq, dtype=np.int64)


def mrope_ids(index: int, batch: int, seq: int, rows: int, oob_fraction: float) -> np.ndarray:
    """(3, B, S) temporal/height/width ids: text spans and 32x32 image grids.

    Per batch, a start position p ~ U[0, 8192); segments of 512 text, one
    1024-token image, 1024 text, one image, 512 text tokens (scaled to S if S
    differs from 4096). A text token has t = h = w = p and advances p by 1; an
    image of g x g patches starting at p0 gives the patch in row r, column c
    the ids (p0, p0 + r, p0 + c) and then sets p = p0 + g. Finally a fraction
    of all 3*B*S entries, picked without replacement, is moved out of
    [0, rows): half negative (-1 - U[0, 2^31)), half at or beyond the table
    (rows + U[0, 2^40), some past 2^31)."""
    gen = SplitMix64(seed(index, 1))
    ids = np.zeros((3, batch, seq), np.int64)
    grid = 32 if seq >= 4096 else max(1, int(np.sqrt(seq // 4)))
    img = grid * grid
    text_total = seq - 2 * img
    t1 = text_total // 4
    t2 = text_total // 2
    t3 = text_total - t1 - t2
    plan = [("text", t1), ("image", img), ("text", t2), ("image", img), ("text", t3)]
    for b in range(batch):
        p = int(gen.below(1, 8192)[0])
        s = 0
        for kind, n in plan:
            if kind == "text":
                ids[:, b, s:s + n] = np.arange(p, p + n, dtype=np.int64)[None, :]
                p += n
                s += n
            else:
                r = np.repeat(np.arange(grid, dtype=np.int64), grid)
                c = np.tile(np.arange(grid, dtype=np.int64), grid)
                ids[0, b, s:s + n] = p
                ids[1, b, s:s + n] = p + r
                ids[2, b, s:s + n] = p + c
                p += grid
                s += n
    n_oob = int(round(oob_fraction * ids.size))
    if n_oob:
        sel = SplitMix64(seed(index, 3))
        flat = ids.reshape(-1)
        picks = sample_without_replacement(sel, flat.size, n_oob)
        for j, pos in enumerate(picks):
            if j % 2 == 0:
                flat[pos] = -1 - sel.below_big(1 << 31)
            else:
                flat[pos] = rows + sel.below_big(1 << 40)
    return ids


WORKLOADS = {
    "c1_rope_f32_tiny": Workload(
        index=0, name="c1_rope_f32_tiny", op="rope", dtype=np.float32,
        x_shape=(1, 2, 16, 8), has_ids=False, cache_base=10000.0,
        description="RotaryEmbedding rank-4 fp32 (1,2,16,8), (1,16,4) per-token table, no ids"),
    "c2_rope_f16_prefill": Workload(
        index=1, name="c2_rope_f16_prefill", op="rope", dtype=np.float16,
        x_shape=(4, 2048, 4096), num_heads=32, cache_rows=8192, cache_base=1e6,
        extra={"ids": "offset_arange", "offset_bound": 4096},
        description="RotaryEmbedding rank-3 fp16 (4,2048,4096), 32 heads of 128, "
                    "ids = per-batch offset + arange, table (8192,64) base 1e6"),
    "c3_rope_f32_partial_interleaved": Workload(
        index=2, name="c3_rope_f32_partial_interleaved", op="rope", dtype=np.float32,
        x_shape=(8, 32, 1024, 96), rotary_embedding_dim=64, interleaved=1,
        cache_rows=4096, cache_base=10000.0, extra={"ids": "uniform", "id_bound": 4096},
        description="RotaryEmbedding rank-4 fp32 (8,32,1024,96), R=64 interleaved, "
                    "tail of 32 passed through, ids U[0,4096), table (4096,32)"),
    "c4_mrope_f16_prefill": Workload(
        index=3, name="c4_mrope_f16_prefill", op="mrope", dtype=np.float16,
        x_shape=(2, 28, 4096, 128), num_heads=28, cache_rows=32768, cache_base=1e6,
        mrope_section=(16, 24, 24), mrope_layout=0, scale=1.0,
        extra={"oob_fraction": 0.01},
        description="MRotaryEmbedding rank-4 fp16 (2,28,4096,128), section [16,24,24], "
                    "text spans + 32x32 image grids, 1% ids out of range, table (32768,64)"),
    "c5_rope_qk_f16_decode": Workload(
        index=4, name="c5_rope_qk_f16_decode", op="rope_qk", dtype=np.float16,
        x_shape=(256, 1, 4096), num_heads=32, k_shape=(256, 1, 1024), kv_num_heads=8,
        cache_rows=32768, cache_base=1e6, extra={"ids": "uniform", "id_bound": 32768},
        description="Decode Q+K fp16: batch 256, seq 1, Q 32 heads + K 8 heads of 128, "
                    "positions U[0,32768), table (32768,64) or on the fly"),
}


# Workloads of the fused variants (same seeding scheme, indices after the five).
EXTRA_WORKLOADS = {
    "qkv_packed_f16_decode": Workload(
        index=5, name="qkv_packed_f16_decode", op="qkv_packed", dtype=np.float16,
        x_shape=(256, 1, 48 * 128), num_heads=32, kv_num_heads=8, cache_rows=32768, cache_base=1e6,
        extra={"ids": "uniform", "id_bound": 32768},
        description="Packed [Q|K|V] decode fp16: batch 256, seq 1, 32 query + 8 key + 8 value heads "
                    "of 128 in one (256, 1, 6144) tensor; Q and K rotated, V copied; table (32768, 64)"),
    "kv_append_f16_decode": Workload(
        index=6, name="kv_append_f16_decode", op="kv_append", dtype=np.float16,
        x_shape=(256, 1, 4096), num_heads=32, k_shape=(256, 1, 1024), kv_num_heads=8,
        cache_rows=32768, cache_base=1e6, extra={"cache_seq": 4096},
        description="Decode fp16 with cache append: batch 256, seq 1, Q 32 heads + K, V 8 heads of 128, "
                    "caches (256, 8, 4096, 128), lengths U[1, 4096], table (32768, 64)"),
}


EXTRA_WORKLOADS.update({
    "qk_norm_f16_prefill": Workload(
        index=7, name="qk_norm_f16_prefill", op="qk_norm", dtype=np.float16,
        x_shape=(4, 2048, 4096), num_heads=32, k_shape=(4, 2048, 1024), kv_num_heads=8,
        cache_rows=8192, cache_base=1e6, extra={"ids": "offset_arange", "offset_bound": 4096},
        description="QK-norm + RoPE prefill fp16 (Qwen3 layout): Q (4, 2048, 32x128), K (4, 2048, 8x128), "
                    "RMSNorm weights (128,), ids = per-batch offset + arange, table (8192, 64) base 1e6"),
    "qk_norm_kv_append_f16_decode": Workload(
        index=9, name="qk_norm_kv_append_f16_decode", op="kv_append_norm", dtype=np.float16,
        x_shape=(256, 1, 4096), num_heads=32, k_shape=(256, 1, 1024), kv_num_heads=8,
        cache_rows=32768, cache_base=1e6, extra={"cache_seq": 4096},
        description="QK-norm model decode step: Q 32 + K, V 8 heads of 128 (batch 256), RMSNorm of Q and "
                    "K, RoPE, K and V appended to (256, 8, 4096, 128) caches, lengths U[1, 4096]"),
    "mrope_f16_decode": Workload(
        index=10, name="mrope_f16_decode", op="mrope", dtype=np.float16,
        x_shape=(256, 1, 28 * 128), num_heads=28, cache_rows=32768, cache_base=1e6,
        mrope_section=(16, 24, 24), mrope_layout=0, scale=1.0, extra={"ids": "decode"},
        description="MRotaryEmbedding decode fp16 (Qwen2-VL-like): batch 256, seq 1, 28 heads of 128, "
                    "rank 3, section [16,24,24], the three streams at the token's position U[0, 32768), "
                    "table (32768, 64)"),
    "qk_norm_f16_decode": Workload(
        index=8, name="qk_norm_f16_decode", op="qk_norm", dtype=np.float16,
        x_shape=(256, 1, 4096), num_heads=32, k_shape=(256, 1, 1024), kv_num_heads=8,
        cache_rows=32768, cache_base=1e6, extra={"ids": "uniform", "id_bound": 32768},
        description="QK-norm + RoPE decode fp16: batch 256, Q 32 + K 8 heads of 128, positions "
                    "U[0, 32768), coefficients on the fly"),
})


# One GPU's share of c2 and c5 under 8-way tensor parallelism (heads split
# over the GPUs, every token on every GPU), and of c2 under 8-way sequence
# parallelism (tokens split, whole rows): the same kernels at the shard's
# real shape.
EXTRA_WORKLOADS.update({
    "c2_rope_f16_prefill_tp8": Workload(
        index=11, name="c2_rope_f16_prefill_tp8", op="rope", dtype=np.float16,
        x_shape=(4, 2048, 512), num_heads=4, cache_rows=8192, cache_base=1e6,
        extra={"ids": "offset_arange", "offset_bound": 4096},
        description="c2's share on one of 8 GPUs (heads split 8 ways): RotaryEmbedding rank-3 fp16 "
                    "(4,2048,512), 4 heads of 128, ids = per-batch offset + arange, table (8192,64) base 1e6"),
    "c5_rope_qk_f16_decode_tp8": Workload(
        index=12, name="c5_rope_qk_f16_decode_tp8", op="rope_qk", dtype=np.float16,
        x_shape=(256, 1, 512), num_heads=4, k_shape=(256, 1, 128), kv_num_heads=1,
        cache_rows=32768, cache_base=1e6, extra={"ids": "uniform", "id_bound": 32768},
        description="c5's share on one of 8 GPUs (heads split 8 ways): decode Q+K fp16, batch 256, "
                    "Q 4 heads + K 1 head of 128, positions U[0,32768), table (32768,64) or on the fly"),
    "kv_append_f16_prompt": Workload(
        index=14, name="kv_append_f16_prompt", op="kv_append", dtype=np.float16,
        x_shape=(4, 2048, 4096), num_heads=32, k_shape=(4, 2048, 1024), kv_num_heads=8,
        cache_rows=8192, cache_base=1e6, extra={"cache_seq": 4096, "prompt": True},
        description="Prompt with cache append fp16: 4 sequences of 2048 new tokens, Q 32 heads + K, V "
                    "8 heads of 128, written to rows 0..2047 of (4, 8, 4096, 128) caches, table (8192, 64)"),
    "c2_rope_f16_prefill_sp8": Workload(
        index=13, name="c2_rope_f16_prefill_sp8", op="rope", dtype=np.float16,
        x_shape=(4, 256, 4096), num_heads=32, cache_rows=8192, cache_base=1e6,
        extra={"ids": "offset_arange", "offset_bound": 7936},
        description="c2's share on one of 8 GPUs (sequence split 8 ways): RotaryEmbedding rank-3 fp16 "
                    "(4,256,4096), 32 heads of 128, ids = per-batch offset U[0,7936) + arange, table (8192,64)"),
})


# Prefills of other model shapes (fp16, 4 x 2048 tokens): small heads, a
# GPT-NeoX-style partial rotation whose pairs do not fall on 16-byte chunks,
# and QK-norm with heads of 256 (Gemma-3-like).
EXTRA_WORKLOADS.update({
    "rope_f16_prefill_heads64": Workload(
        index=15, name="rope_f16_prefill_heads64", op="rope", dtype=np.float16,
        x_shape=(4, 2048, 64 * 64), num_heads=64, cache_rows=8192, cache_base=1e4,
        extra={"ids": "offset_arange", "offset_bound": 4096},
        description="RotaryEmbedding rank-3 fp16 (4,2048,4096), 64 heads of 64, ids = per-batch offset + "
                    "arange, table (8192,32) base 1e4"),
    "rope_f16_prefill_neox_partial": Workload(
        index=16, name="rope_f16_prefill_neox_partial", op="rope", dtype=np.float16,
        x_shape=(4, 2048, 64 * 96), num_heads=64, rotary_embedding_dim=24, cache_rows=8192,
        cache_base=1e4, extra={"ids": "offset_arange", "offset_bound": 4096},
        description="RotaryEmbedding rank-3 fp16 (4,2048,6144), 64 heads of 96 with the first 24 "
                    "dimensions rotated (GPT-NeoX-20B's shape), ids = per-batch offset + arange, table (8192,12)"),
    "qk_norm_f16_prefill_heads256": Workload(
        index=17, name="qk_norm_f16_prefill_heads256", op="qk_norm", dtype=np.float16,
        x_shape=(4, 2048, 8 * 256), num_heads=8, k_shape=(4, 2048, 4 * 256), kv_num_heads=4,
        cache_rows=8192, cache_base=1e6, extra={"ids": "offset_arange", "offset_bound": 4096},
        description="QK-norm + RoPE prefill fp16 with heads of 256 (Gemma-3-like): Q (4,2048,8x256), "
                    "K (4,2048,4x256), ids = per-batch offset + arange, table (8192,128) base 1e6"),
})


def get(name: str) -> Workload:
    return WORKLOADS[name] if name in WORKLOADS else EXTRA_WORKLOADS[name]


def normal_like_type(v: np.ndarray, dtype) -> np.ndarray:
    """binary32 values rounded to `dtype` (bfloat16 as uint16 bits)."""
    from .generators import BFLOAT16, bfloat16_bits
    if np.dtype(dtype) == BFLOAT16:
        return bfloat16_bits(v)
    return v.astype(dtype)


def with_dtype(w: Workload, dtype, tag: str) -> Workload:
    """The same workload stored in another type (same seeds and structure)."""
    from dataclasses import replace
    return replace(w, dtype=dtype, name="%s_%s" % (w.name, tag))


def with_layout(w: Workload, layout: int) -> Workload:
    from dataclasses import replace
    return replace(w, mrope_layout=layout, name="%s_layout%d" % (w.name.rsplit("_layout", 1)[0], layout))
