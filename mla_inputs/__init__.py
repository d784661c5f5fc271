"""Seeded synthetic inputs for the MLA decode step (data only).

This module is the one piece of code that both the CPU oracle and the HIP path
use: it draws random numbers, stores them in the input number formats and lays
out the sequence structure (lengths, positions, page tables).  It holds none of
the attention method's arithmetic: no projection, no RoPE, no softmax and no
quantisation.  It never imports the oracle or the HIP package.

Shapes follow the MLA hyper-parameters of "DeepSeek-V2: Strong, Economical,
Efficient" (section 3.2.1: n_h = 128 heads, d_h = 128, d_c = 512, d_h^R = 64)
and the "DeepSeek-V3 Technical Report" notes (MLA section, same dimensions).

Draw recipe (every workload):
  * ``numpy.random.SeedSequence(seed).spawn(9)`` gives one independent stream
    per field, in this fixed order: W_UK, W_UV, q_nope, q_rope, c_KV, k_R,
    lengths, page permutation, outlier picks.  Because each field has its own
    stream, a field's values do not depend on the sizes of the other fields.
  * Gaussian fields are drawn as float32 ``standard_normal`` and multiplied by
    their standard deviation in float32 (W ~ N(0, 1/d_c): variance 1/d_c).
  * bf16 fields are then rounded to bfloat16 with round-to-nearest-even and
    kept as their 16-bit patterns (``numpy.uint16``); fp32 fields stay float32.
  * Lengths (paged workload): L_b = round(exp(U[ln lo, ln hi])).
  * Pages (paged workload): sequence b owns ceil(L_b / page) pages; one random
    permutation of all page ids is handed out in sequence order.  Unused
    page-table entries hold -1 and are never read.
  * Outliers (long-context workload): round(frac * L) distinct token rows per
    sequence, uniform without replacement; only the c_KV row is multiplied by
    the outlier factor (a power of two, so exact in bf16).
  * fp8- and 6-bit-cache workloads: the c_KV / k_R rows generated here are
    the bf16 source rows that the cache-append step quantises; quantisation is
    not done here.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "generate", "bf16_bits_from_f32",
           "kv_row_layout"]

FIELDS = ("w_uk", "w_uv", "q_nope", "q_rope", "c_kv", "k_r",
          "lengths", "pages", "outliers")


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode workload.

    ``kv_len`` is the KV length of every sequence *including* the T query
    tokens, which are already in the cache when the step runs.
    """
    name: str
    batch: int
    q_tokens: int              # T query tokens per sequence (causal)
    n_heads: int
    d_head: int
    d_latent: int
    d_rope: int
    kv_len: int = 0            # uniform length; 0 when len_range is used
    len_range: Tuple[int, int] = (0, 0)   # log-uniform [lo, hi]
    lengths: Tuple[int, ...] = ()          # explicit per-sequence lengths
    kv_dtype: str = "bf16"     # "f32" | "bf16" | "fp8" | "fp6"
    q_dtype: str = "bf16"      # "f32" | "bf16"
    layout: str = "contiguous"  # "contiguous" | "paged"
    page_size: int = 64
    rope: bool = False         # True: q_R / k_R are raw and RoPE is applied
    rope_base: float = 10000.0
    num_splits: int = 0        # 0: let the library choose
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    seed: int = 0
    description: str = ""
    d_model: int = 5120        # hidden size d (rows of W^O)
    # context extension of the RoPE parts (YaRN); yarn_factor <= 1: off
    yarn_factor: float = 0.0   # s
    yarn_alpha: float = 1.0
    yarn_beta: float = 32.0
    yarn_orig_len: int = 4096  # original (training) context
    yarn_coef: float = 0.0707  # sqrt(t) = coef * ln(s) + 1

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload(
            name="tiny_fp32", batch=1, q_tokens=1, n_heads=4, d_head=16,
            d_latent=32, d_rope=16, kv_len=64, kv_dtype="f32", q_dtype="f32",
            rope=True, d_model=48,
            description="Tiny MLA decode, fp32: B=1, T=1, n_h=4, d_h=16, "
                        "d_c=32, d_h^R=16, L=64, RoPE base 1e4 at positions "
                        "0..63"),
        Workload(
            name="v2_b32_l4k_bf16", batch=32, q_tokens=1, n_heads=128,
            d_head=128, d_latent=512, d_rope=64, kv_len=4096,
            description="DeepSeek-V2 MLA layer decode, bf16: B=32, T=1, "
                        "n_h=128, L=4096, contiguous latent cache"),
        Workload(
            name="v2_paged_b128_bf16", batch=128, q_tokens=1, n_heads=128,
            d_head=128, d_latent=512, d_rope=64, len_range=(512, 32768),
            layout="paged",
            description="Paged batched decode, bf16: B=128, KV lengths "
                        "log-uniform in [512, 32768], 64-token pages, "
                        "shuffled page table"),
        Workload(
            name="v2_long_b4_l128k_bf16", batch=4, q_tokens=1, n_heads=128,
            d_head=128, d_latent=512, d_rope=64, kv_len=131072, num_splits=64,
            outlier_frac=0.01, outlier_scale=8.0,
            description="Long-context split-KV decode, bf16: B=4, L=131072, "
                        "64 KV chunks + LSE combine, 1% of c_KV rows x8"),
        Workload(
            name="v2_fp8_t4_b64_l8k", batch=64, q_tokens=4, n_heads=128,
            d_head=128, d_latent=512, d_rope=64, kv_len=8192, kv_dtype="fp8",
            description="fp8 e4m3 latent cache (per-token fp32 scale) + "
                        "4 causal query tokens: B=64, T=4, L=8192"),
        Workload(
            name="v2_fp6_t4_b64_l8k", batch=64, q_tokens=4, n_heads=128,
            d_head=128, d_latent=512, d_rope=64, kv_len=8192, kv_dtype="fp6",
            description="6-bit latent cache (E2M3 codes, one E8M0 power of two "
                        "per 32 elements) + 4 causal query tokens: B=64, T=4, "
                        "L=8192"),
        Workload(
            name="v2_b64_l8k_bf16", batch=64, q_tokens=1, n_heads=128,
            d_head=128, d_latent=512, d_rope=64, kv_len=8192,
            description="bf16 companion of the fp8 workload: B=64, T=1, "
                        "L=8192, contiguous"),
        Workload(
            name="v2lite_b64_l8k_bf16", batch=64, q_tokens=1, n_heads=16,
            d_head=128, d_latent=512, d_rope=64, kv_len=8192, d_model=2048,
            description="DeepSeek-V2-Lite attention shapes (16 heads, hidden "
                        "size 2048), bf16: B=64, T=1, L=8192, contiguous"),
    ]
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def _gauss(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    if dtype == "f32":
        return x
    return bf16_bits_from_f32(x)


def kv_row_layout(w: Workload, seq_lens: np.ndarray):
    """Sequence structure of the cache rows: (row_offsets, row_seq, row_pos).

    The rows of all sequences are concatenated in sequence order; row r of the
    concatenation belongs to sequence row_seq[r] at token position row_pos[r].
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    offsets = np.zeros(len(seq_lens) + 1, dtype=np.int64)
    np.cumsum(seq_lens, out=offsets[1:])
    total = int(offsets[-1])
    row_seq = np.repeat(np.arange(len(seq_lens), dtype=np.int32), seq_lens)
    row_pos = (np.arange(total, dtype=np.int64) - offsets[row_seq]).astype(np.int32)
    return offsets, row_seq, row_pos


def generate(w: Workload, seed: Optional[int] = None,
             with_cache_rows: bool = True) -> Dict[str, np.ndarray]:
    """Draw every input of one decode step of workload ``w``.

    Returns a dict of numpy arrays (bf16 fields as uint16 bit patterns):
      w_uk, w_uv   [n_h, d_h, d_c]    head i = rows [i*d_h, (i+1)*d_h) of W
      q_nope       [B*T, n_h, d_h]    q^C per query token (b-major, then tau)
      q_rope       [B*T, n_h, d_h^R]  q^R (raw when ``w.rope``, else rotated)
      c_kv         [sum L, d_c]       latent rows, sequences concatenated
      k_r          [sum L, d_h^R]     shared RoPE key rows (raw when ``w.rope``)
      seq_lens     [B] int32          KV length incl. the T query tokens
      row_offsets  [B+1] int64, row_seq [sum L] int32, row_pos [sum L] int32
      q_pos        [B*T] int32        position of each query token
      page_table   [B, max_pages] int32 (paged layout only)
    """
    seed = w.seed if seed is None else seed
    streams = dict(zip(FIELDS, np.random.SeedSequence(seed).spawn(len(FIELDS))))
    rng = {k: np.random.default_rng(s) for k, s in streams.items()}
    B, T, H = w.batch, w.q_tokens, w.n_heads
    wdt = "f32" if w.q_dtype == "f32" else "bf16"
    src_dt = "f32" if w.kv_dtype == "f32" else "bf16"
    wstd = 1.0 / math.sqrt(w.d_latent)

    out: Dict[str, np.ndarray] = {}
    out["w_uk"] = _gauss(rng["w_uk"], (H, w.d_head, w.d_latent), wstd, wdt)
    out["w_uv"] = _gauss(rng["w_uv"], (H, w.d_head, w.d_latent), wstd, wdt)
    out["q_nope"] = _gauss(rng["q_nope"], (B * T, H, w.d_head), 1.0, w.q_dtype)
    out["q_rope"] = _gauss(rng["q_rope"], (B * T, H, w.d_rope), 1.0, w.q_dtype)

    if w.lengths:
        if len(w.lengths) != B:
            raise ValueError("lengths must list one length per sequence")
        seq_lens = np.asarray(w.lengths, dtype=np.int32)
    elif w.kv_len > 0:
        seq_lens = np.full(B, w.kv_len, dtype=np.int32)
    else:
        lo, hi = w.len_range
        u = rng["lengths"].uniform(math.log(lo), math.log(hi), size=B)
        seq_lens = np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)
    if np.any(seq_lens < T):
        raise ValueError("every sequence must hold at least T tokens")
    out["seq_lens"] = seq_lens
    offsets, row_seq, row_pos = kv_row_layout(w, seq_lens)
    out["row_offsets"], out["row_seq"], out["row_pos"] = offsets, row_seq, row_pos
    q_pos = (seq_lens[:, None] - T + np.arange(T)[None, :]).reshape(-1)
    out["q_pos"] = q_pos.astype(np.int32)

    total = int(offsets[-1])
    if with_cache_rows:
        if w.outlier_frac > 0.0:
            c = rng["c_kv"].standard_normal(size=(total, w.d_latent), dtype=np.float32)
            n_out = int(round(w.outlier_frac * int(seq_lens[0]))) if w.kv_len else None
            for b in range(B):
                L = int(seq_lens[b])
                k = n_out if n_out is not None else int(round(w.outlier_frac * L))
                picks = rng["outliers"].choice(L, size=k, replace=False)
                c[offsets[b] + picks] *= np.float32(w.outlier_scale)
            out["c_kv"] = c if src_dt == "f32" else bf16_bits_from_f32(c)
        else:
            out["c_kv"] = _gauss(rng["c_kv"], (total, w.d_latent), 1.0, src_dt)
        out["k_r"] = _gauss(rng["k_r"], (total, w.d_rope), 1.0, src_dt)

    if w.layout == "paged":
        P = w.page_size
        n_pages = (seq_lens.astype(np.int64) + P - 1) // P
        max_pages = int(n_pages.max())
        perm = rng["pages"].permutation(int(n_pages.sum())).astype(np.int32)
        table = np.full((B, max_pages), -1, dtype=np.int32)
        start = 0
        for b in range(B):
            table[b, :n_pages[b]] = perm[start:start + n_pages[b]]
            start += int(n_pages[b])
        out["page_table"] = table
        out["num_pages"] = np.int64(n_pages.sum())
    return out


def output_weights(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """W^O [d_model, n_h * d_h] (the attention output projection), drawn
    from its own stream (child len(FIELDS) of the workload's seed, so that
    no other field changes): N(0, 1/(n_h d_h)), rounded like W^UK / W^UV."""
    seed = w.seed if seed is None else seed
    ss = np.random.SeedSequence(seed).spawn(len(FIELDS) + 1)[len(FIELDS)]
    K = w.n_heads * w.d_head
    wdt = "f32" if w.q_dtype == "f32" else "bf16"
    return _gauss(np.random.default_rng(ss), (w.d_model, K), 1.0 / math.sqrt(K), wdt)


def producer_inputs(w: Workload, n_rows: int, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of the cache producer, from their own stream (child
    len(FIELDS) + 1 of the workload's seed): hidden states h [n_rows, d_model]
    ~ N(0, 1); [W^DKV; W^KR] [d_c + d_h^R, d_model] ~ N(0, 1/d_model) (unit-
    variance outputs), both rounded like the queries / weights; an RMS-norm
    gain [d_c] ~ N(1, 0.1^2) in fp32."""
    seed = w.seed if seed is None else seed
    ss = np.random.SeedSequence(seed).spawn(len(FIELDS) + 2)[len(FIELDS) + 1]
    rng = np.random.default_rng(ss)
    wdt = "f32" if w.q_dtype == "f32" else "bf16"
    D = w.d_latent + w.d_rope
    return {
        "h": _gauss(rng, (n_rows, w.d_model), 1.0, w.q_dtype),
        "w_dkv_kr": _gauss(rng, (D, w.d_model), 1.0 / math.sqrt(w.d_model), wdt),
        "gain": (1.0 + 0.1 * rng.standard_normal(w.d_latent)).astype(np.float32),
    }


def small_variant(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields changed (used for scaled-down tests)."""
    return dataclasses.replace(w, **changes)
