"""The MLA decode step, literal and un-absorbed (oracle; test infrastructure).

Sources (cited by page title and section / equation):
  [V2]  "DeepSeek-V2: Strong, Economical, Efficient": section 2.1.2 (low-rank
        key-value joint compression: only c^KV is cached, W^UK and W^UV are
        the d_h n_h x d_c up-projections), section 2.1.3 (decoupled RoPE: one
        shared k^R per token, cached next to c^KV; per-head q^R), Appendix C
        (full formulas; the naive form recovers k^C and v^C from c^KV).
  [V3]  "DeepSeek-V3 Technical Report" notes, MLA section: the equations
        k^C_t = W^UK c^KV_t split into n_h head blocks, k_{t,i} = [k^C_{t,i};
        k^R_t], v^C_t = W^UV c^KV_t, q_{t,i} = [q^C_{t,i}; q^R_{t,i}], and the
        attention-output equation
            o_{t,i} = sum_{j=1..t} Softmax_j(q_{t,i}^T k_{j,i} / sqrt(d_h + d_h^R)) v^C_{j,i}.

Readings where the pages leave a step open:
  * The sum runs over j = 1..t, so the current token is included: a query
    token at position p (0-based) attends to cache rows 0..p.  With T query
    tokens per sequence of KV length L (the T tokens already cached), query
    tau sits at position L - T + tau.
  * W^UK, W^UV in R^{d_h n_h x d_c}: head i owns rows [i d_h, (i+1) d_h).  They
    are stored as [n_h, d_h, d_c].
  * The cache row of a token is [c^KV (d_c) | k^R (d_h^R)], k^R already
    rotated.
  * Besides o, the oracle returns the latent-space weighted sum
    sum_j p_j c_j and the natural-log LSE of the scores, so the attention
    stage can be checked on its own.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np

from . import formats
from .rope import rope as _rope
from .rope import yarn_logit_factor, yarn_theta


def attend_head(q_c: np.ndarray, q_r: np.ndarray, C: np.ndarray, KR: np.ndarray,
                w_uk_i: np.ndarray, w_uv_i: np.ndarray, scale: float):
    """One head, one query, over cache rows C [n, d_c], KR [n, d_h^R].

    Keys and values are materialised per head, exactly as written in [V3]:
    k_j = [W^UK_i c_j ; k^R_j], v_j = W^UV_i c_j.
    Returns (o [d_h], latent [d_c], lse).
    """
    K_c = C @ w_uk_i.T                       # [n, d_h]   k^C_{j,i}
    K = np.concatenate([K_c, KR], axis=1)    # [n, d_h + d_h^R]
    V = C @ w_uv_i.T                         # [n, d_h]   v^C_{j,i}
    q = np.concatenate([q_c, q_r])           # [d_h + d_h^R]
    s = (K @ q) * scale
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    p = e / z
    return p @ V, p @ C, m + math.log(z)


def decode(q_nope: np.ndarray, q_rope: np.ndarray, w_uk: np.ndarray,
           w_uv: np.ndarray, c_rows: np.ndarray, kr_rows: np.ndarray,
           row_offsets: np.ndarray, seq_lens: np.ndarray, q_tokens: int,
           softmax_scale: Optional[float] = None,
           seqs: Optional[Iterable[int]] = None,
           heads: Optional[Iterable[int]] = None) -> Dict[str, np.ndarray]:
    """Literal MLA decode for query tokens n = b*T + tau (float64).

    q_nope [B*T, n_h, d_h], q_rope [B*T, n_h, d_h^R] (already rotated),
    w_uk / w_uv [n_h, d_h, d_c], c_rows [sum L, d_c], kr_rows [sum L, d_h^R]
    (sequence b owns rows row_offsets[b] : row_offsets[b] + seq_lens[b]).
    ``seqs`` / ``heads`` restrict the work to a sample; entries outside the
    sample are NaN in the outputs.
    """
    n_tok, H, d_h = q_nope.shape
    d_r = q_rope.shape[2]
    d_c = w_uk.shape[2]
    T = q_tokens
    B = len(seq_lens)
    if n_tok != B * T:
        raise ValueError("q_nope must hold B*T query tokens")
    scale = 1.0 / math.sqrt(d_h + d_r) if softmax_scale is None else softmax_scale
    seqs = range(B) if seqs is None else list(seqs)
    heads = range(H) if heads is None else list(heads)
    o = np.full((n_tok, H, d_h), np.nan)
    lat = np.full((n_tok, H, d_c), np.nan)
    lse = np.full((n_tok, H), np.nan)
    for b in seqs:
        L = int(seq_lens[b])
        if L < T or L < 1:
            raise ValueError("a decode step needs L >= T >= 1")
        r0 = int(row_offsets[b])
        C = np.asarray(c_rows[r0:r0 + L], dtype=np.float64)
        KR = np.asarray(kr_rows[r0:r0 + L], dtype=np.float64)
        for tau in range(T):
            n = b * T + tau
            p_q = L - T + tau                  # position of this query token
            for i in heads:
                o[n, i], lat[n, i], lse[n, i] = attend_head(
                    q_nope[n, i], q_rope[n, i], C[:p_q + 1], KR[:p_q + 1],
                    w_uk[i], w_uv[i], scale)
    return {"o": o, "latent": lat, "lse": lse}


def absorbed_query(q_nope: np.ndarray, q_rope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """The absorbed query of [V2] Appendix C: by associativity,
    q^C_i . (W^UK_i c) = (W^UK_i^T q^C_i) . c, so the per-head query against
    the cache row [c ; k^R] is [W^UK_i^T q^C_i ; q^R_i].

    q_nope [N, n_h, d_h], q_rope [N, n_h, d_h^R] (rotated), w_uk [n_h, d_h, d_c]
    -> [N, n_h, d_c + d_h^R] (float64).
    """
    n_tok, H, _ = q_nope.shape
    out = np.empty((n_tok, H, w_uk.shape[2] + q_rope.shape[2]))
    for i in range(H):
        out[:, i, :w_uk.shape[2]] = q_nope[:, i, :] @ w_uk[i]
        out[:, i, w_uk.shape[2]:] = q_rope[:, i, :]
    return out


def up_project(latent: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """o_{n,i} = W^UV_i latent_{n,i}: the value up-projection applied after
    the latent-space weighted sum ([V2] Appendix C; exact because
    sum_j p_j W^UV_i c_j = W^UV_i sum_j p_j c_j).

    latent [N, n_h, d_c], w_uv [n_h, d_h, d_c] -> [N, n_h, d_h] (float64).
    """
    n_tok, H, _ = latent.shape
    out = np.empty((n_tok, H, w_uv.shape[1]))
    for i in range(H):
        out[:, i, :] = latent[:, i, :] @ w_uv[i].T
    return out


def produce_rows(h: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray, gain, eps: float,
                 pos=None, rope_base: float = 10000.0, theta=None) -> np.ndarray:
    """The cache row of each token, from its hidden state h_t ([V3] notes, MLA
    section: c^KV_t = W^DKV h_t and k^R_t = RoPE(W^KR h_t); [V2] section 3.2.1:
    an RMS norm follows the compressed latent vector):
        c = W^DKV h,  c <- c * gain / sqrt(mean(c^2) + eps)  (gain None: no norm),
        k = W^KR h, rotated at position pos (pos None: not rotated) by the
            frequencies theta (None: plain RoPE with rope_base),
        row = [c ; k].

    h [N, d], w_dkv [d_c, d], w_kr [d_h^R, d], gain [d_c] or None, pos [N]
    -> [N, d_c + d_h^R] (float64).
    """
    c = h @ w_dkv.T
    if gain is not None:
        rms = np.sqrt(np.mean(c * c, axis=1, keepdims=True) + eps)
        c = c / rms * np.asarray(gain, dtype=np.float64)[None, :]
    k = h @ w_kr.T
    if pos is not None:
        k = _rope(k, np.asarray(pos), rope_base, theta=theta)
    return np.concatenate([c, k], axis=1)


def output_project(o: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """u_n = W^O [o_{n,1}; o_{n,2}; ...; o_{n,n_h}]: the attention output
    projection of the [V3] notes, MLA section (the equation after the
    attention-output equation), W^O in R^{d x d_h n_h}.  Written per head
    block: column block i of W^O (columns [i d_h, (i+1) d_h)) multiplies
    o_{n,i}, and the blocks are summed.

    o [N, n_h, d_h], w_o [d, n_h d_h] -> u [N, d] (float64).
    """
    n_tok, H, d_h = o.shape
    u = np.zeros((n_tok, w_o.shape[0]))
    for i in range(H):
        u += o[:, i, :] @ w_o[:, i * d_h:(i + 1) * d_h].T
    return u


def _to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return formats.bf16_to_f64(a)
    raise ValueError(dtype)


def logical_inputs(gen: Dict[str, np.ndarray], workload, seqs=None) -> Dict[str, np.ndarray]:
    """Decode the generator's stored inputs into the oracle's float64 operands.

    Applies the steps that precede attention in the method, the oracle's way:
      * RoPE on q^R at the query positions and on k^R at the row positions
        when the workload carries raw (unrotated) RoPE parts;
      * for the fp8 cache, the per-token E4M3 quantisation of the source rows
        (float32 decisions, see ``formats``), for the 6-bit cache the E2M3
        quantisation with one shared power of two per 32 elements, each
        followed by exact dequantisation: the dequantised cache *is* the
        attention input.
    ``seqs`` limits the cache rows decoded to those sequences (the returned
    row_offsets then index the compacted rows).
    """
    w = workload
    d = {
        "w_uk": _to_f64(gen["w_uk"], "f32" if w.q_dtype == "f32" else "bf16"),
        "w_uv": _to_f64(gen["w_uv"], "f32" if w.q_dtype == "f32" else "bf16"),
        "q_nope": _to_f64(gen["q_nope"], w.q_dtype),
        "q_rope": _to_f64(gen["q_rope"], w.q_dtype),
        "seq_lens": gen["seq_lens"],
        "row_offsets": gen["row_offsets"],
    }
    src_dt = "f32" if w.kv_dtype == "f32" else "bf16"
    offs = np.asarray(gen["row_offsets"], dtype=np.int64)
    if seqs is None:
        idx = slice(None)
        row_pos = gen["row_pos"]
    else:
        seqs = sorted(set(int(b) for b in seqs))
        idx = np.concatenate([np.arange(offs[b], offs[b + 1]) for b in seqs])
        row_pos = gen["row_pos"][idx]
        new_offs = np.zeros_like(offs)
        start = 0
        for b in seqs:
            new_offs[b] = start
            start += offs[b + 1] - offs[b]
        d["row_offsets"] = new_offs
    c = _to_f64(gen["c_kv"][idx], src_dt)
    kr = _to_f64(gen["k_r"][idx], src_dt)
    if w.rope:
        theta = yarn_theta(w.d_rope, w.rope_base, w.yarn_factor, w.yarn_alpha, w.yarn_beta,
                           w.yarn_orig_len)
        kr = _rope(kr, row_pos, theta=theta)
        qpos = np.repeat(gen["q_pos"], w.n_heads).reshape(-1, w.n_heads)
        d["q_rope"] = _rope(d["q_rope"], qpos, theta=theta)
    if w.kv_dtype == "fp8":
        rows = np.concatenate([c, kr], axis=1).astype(np.float32)
        codes, scales = formats.quantize_rows_e4m3(rows)
        deq = formats.dequantize_rows_e4m3(codes, scales)
        c, kr = deq[:, :w.d_latent], deq[:, w.d_latent:]
        d["fp8_codes"], d["fp8_scales"] = codes, scales
    elif w.kv_dtype == "fp6":
        rows = np.concatenate([c, kr], axis=1).astype(np.float32)
        codes, exps = formats.quantize_rows_mxfp6(rows)
        deq = formats.dequantize_rows_mxfp6(codes, exps)
        c, kr = deq[:, :w.d_latent], deq[:, w.d_latent:]
        d["fp6_codes"], d["fp6_exps"] = codes, exps
    d["c_rows"], d["kr_rows"] = c, kr
    return d


def decode_workload(gen: Dict[str, np.ndarray], workload, seqs=None, heads=None):
    """Oracle outputs for a generated workload (optionally a sample of it)."""
    w = workload
    d = logical_inputs(gen, w, seqs)
    scale = yarn_logit_factor(w.yarn_factor, w.yarn_coef) / math.sqrt(w.d_head + w.d_rope)
    return decode(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["c_rows"],
                  d["kr_rows"], d["row_offsets"], d["seq_lens"],
                  w.q_tokens, softmax_scale=scale, seqs=seqs, heads=heads)


def cache_row_index(seq: np.ndarray, pos: np.ndarray, page_table, page_size: int,
                    max_len: int) -> np.ndarray:
    """Row of the cache buffer that holds token ``pos`` of sequence ``seq``.

    Contiguous layout ([B, max_len, D]): seq * max_len + pos.
    Paged layout ([pages, page_size, D]): page_table[seq, pos // page_size]
    * page_size + pos % page_size.
    """
    seq = np.asarray(seq, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    if page_table is None:
        return seq * max_len + pos
    pt = np.asarray(page_table, dtype=np.int64)
    return pt[seq, pos // page_size] * page_size + pos % page_size
