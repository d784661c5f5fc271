"""ctypes binding of libmla.so (argument marshalling only).

Each function takes torch tensors that live on the GPU (torch provides the
device memory and the stream), passes their raw pointers to the C ABI
declared in include/mla.h, and raises MLAError on a negative status.  All
computation happens in the HIP kernels of libmla.so; if the library is not
built, loading fails with an error instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla.so")

F32, BF16, FP8_E4M3, FP6_E2M3 = 0, 1, 2, 3
DTYPE_CODES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "fp6": FP6_E2M3}
FP6_ROW_BYTES = 452            # bytes per 6-bit cache row of 576 elements
PREC_AUTO, PREC_FP32, PREC_BF16, PREC_BF16X2 = 0, 1, 2, 3
PRECISION_CODES = {"auto": PREC_AUTO, "fp32": PREC_FP32, "bf16": PREC_BF16,
                   "bf16x2": PREC_BF16X2}

EXPORTED = ("mla_absorb_q", "mla_cache_append", "mla_decode_workspace_size",
            "mla_decode_attn", "mla_decode_attn_noalloc", "mla_up_proj_v", "mla_out_proj_workspace_size", "mla_out_proj",
            "mla_kv_produce_workspace_size", "mla_kv_produce",
            "mla_out_proj_pack", "mla_out_proj_packed", "mla_check_page_table",
            "mla_absorb_append",
            "mla_status_string", "mla_version")


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class MLADims(ctypes.Structure):
    """mirror of mla_dims_t"""
    _fields_ = [
        ("n_heads", ctypes.c_int32), ("d_head", ctypes.c_int32),
        ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("rope_base", ctypes.c_float), ("precision", ctypes.c_int32),
        ("yarn_factor", ctypes.c_float), ("yarn_alpha", ctypes.c_float),
        ("yarn_beta", ctypes.c_float), ("yarn_orig_len", ctypes.c_int32),
        ("yarn_coef", ctypes.c_float),
    ]

    @classmethod
    def make(cls, n_heads, d_head, d_latent, d_rope, kv_dtype="bf16",
             q_dtype="bf16", softmax_scale=0.0, rope_base=0.0, page_size=64,
             precision="auto", yarn_factor=0.0, yarn_alpha=1.0, yarn_beta=32.0,
             yarn_orig_len=4096, yarn_coef=0.0707):
        kv = DTYPE_CODES[kv_dtype] if isinstance(kv_dtype, str) else kv_dtype
        qd = DTYPE_CODES[q_dtype] if isinstance(q_dtype, str) else q_dtype
        pr = PRECISION_CODES[precision] if isinstance(precision, str) else precision
        return cls(n_heads, d_head, d_latent, d_rope, page_size, kv, qd,
                   softmax_scale, rope_base, pr, yarn_factor, yarn_alpha, yarn_beta,
                   yarn_orig_len, yarn_coef)

    @classmethod
    def from_workload(cls, w, precision="auto"):
        return cls.make(w.n_heads, w.d_head, w.d_latent, w.d_rope, w.kv_dtype,
                        w.q_dtype, 0.0, w.rope_base, w.page_size, precision,
                        w.yarn_factor, w.yarn_alpha, w.yarn_beta, w.yarn_orig_len,
                        w.yarn_coef)

    def qabs_is_f32(self) -> bool:
        return self.q_dtype == F32 or self.precision == PREC_FP32

    def qabs_pairs(self) -> bool:
        """q_abs holds (hi, lo) bf16 pairs per row (the layout rule of
        mla_absorb_q in include/mla.h)."""
        shape = (self.d_head == 128 and self.d_latent == 512 and self.d_rope == 64
                 and self.q_dtype == BF16 and self.n_heads % 128 == 0)
        return shape and (self.precision == PREC_BF16X2 or
                          (self.precision == PREC_AUTO and self.kv_dtype == BF16))


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m head_latent_attention_11_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pdims = ctypes.POINTER(MLADims)
    lib.mla_absorb_q.argtypes = [pdims, vp, vp, vp, vp, vp, i32, vp]
    lib.mla_cache_append.argtypes = [pdims, vp, vp, vp, vp, vp, i32, i32, i32, i64,
                                     i32, vp, vp, i32, vp]
    lib.mla_decode_workspace_size.argtypes = [pdims, vp, i32, i32, i32,
                                              ctypes.POINTER(sz)]
    lib.mla_decode_attn.argtypes = [pdims, vp, vp, vp, vp, i32, i32, vp, vp, i32, i32,
                                    i32, vp, sz, vp, vp, vp]
    lib.mla_decode_attn_noalloc.argtypes = [pdims, vp, vp, vp, vp, i32, i32, vp, vp, i32, i32,
                                            i32, vp, vp, vp]
    lib.mla_up_proj_v.argtypes = [pdims, vp, vp, vp, i32, i32, vp]
    lib.mla_out_proj_workspace_size.argtypes = [pdims, i32, i32, i32, ctypes.POINTER(sz)]
    lib.mla_out_proj.argtypes = [pdims, vp, i32, vp, i32, vp, i32, i32, vp, sz, vp]
    lib.mla_out_proj_pack.argtypes = [pdims, vp, i32, vp, vp]
    lib.mla_out_proj_packed.argtypes = [pdims, vp, vp, i32, vp, i32, i32, vp, sz, vp]
    lib.mla_kv_produce_workspace_size.argtypes = [pdims, i32, i32, ctypes.POINTER(sz)]
    lib.mla_kv_produce.argtypes = [pdims, vp, i32, vp, vp, ctypes.c_float, vp, vp, vp, i32, i32,
                                   i32, i64, i32, vp, vp, i32, vp, sz, vp]
    lib.mla_status_string.argtypes = [i32]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_check_page_table.argtypes = [pdims, vp, i32, vp, i32, i64, vp, vp]
    lib.mla_absorb_append.argtypes = [pdims, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, i32,
                                      i32, i32, i64, i32, vp, vp, i32, vp]
    lib.mla_version.argtypes = []
    for f in EXPORTED:
        if f not in ("mla_status_string",):
            getattr(lib, f).restype = i32
    lib.mla_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mla_status_string(int(status)).decode()


def version() -> int:
    return int(load_library().mla_version())


def _ptr(t) -> Optional[int]:
    """Raw device pointer of a tensor (None stays NULL; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmla must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream) if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise MLAError(int(status), where)


def absorb_q(dims: MLADims, q_nope, q_rope, w_uk, q_pos, q_abs, n_tokens: int,
             stream=None):
    lib = load_library()
    _check(lib.mla_absorb_q(ctypes.byref(dims), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                            _ptr(q_pos), _ptr(q_abs), int(n_tokens), _stream(stream)),
           "mla_absorb_q")


def cache_append(dims: MLADims, new_c, new_kr, seq_idx, pos, page_table, batch: int,
                 max_pages: int, max_len: int, cache_rows: int, apply_rope: bool,
                 cache, kv_scale, n_rows: int, stream=None):
    lib = load_library()
    _check(lib.mla_cache_append(ctypes.byref(dims), _ptr(new_c), _ptr(new_kr),
                                _ptr(seq_idx), _ptr(pos), _ptr(page_table), int(batch),
                                int(max_pages), int(max_len), int(cache_rows),
                                int(bool(apply_rope)), _ptr(cache), _ptr(kv_scale),
                                int(n_rows), _stream(stream)),
           "mla_cache_append")


def _lens_host(seq_lens_host: Sequence[int]):
    arr = (ctypes.c_int32 * len(seq_lens_host))(*[int(x) for x in seq_lens_host])
    return arr


def decode_workspace_size(dims: MLADims, seq_lens_host: Sequence[int], q_tokens: int,
                          num_splits: int = 0) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    lens = _lens_host(seq_lens_host)
    _check(lib.mla_decode_workspace_size(ctypes.byref(dims), ctypes.cast(lens, ctypes.c_void_p),
                                         len(seq_lens_host), int(q_tokens), int(num_splits),
                                         ctypes.byref(out)),
           "mla_decode_workspace_size")
    return int(out.value)


def decode_attn(dims: MLADims, q_abs, cache, kv_scale, page_table, max_pages: int,
                max_len: int, seq_lens, seq_lens_host: Sequence[int], q_tokens: int,
                num_splits: int, workspace, ws_bytes: int, out_latent, out_lse,
                stream=None, _lens_cache=None):
    lib = load_library()
    lens = _lens_cache if _lens_cache is not None else _lens_host(seq_lens_host)
    _check(lib.mla_decode_attn(ctypes.byref(dims), _ptr(q_abs), _ptr(cache), _ptr(kv_scale),
                               _ptr(page_table), int(max_pages), int(max_len), _ptr(seq_lens),
                               ctypes.cast(lens, ctypes.c_void_p), len(seq_lens_host),
                               int(q_tokens), int(num_splits), _ptr(workspace), int(ws_bytes),
                               _ptr(out_latent), _ptr(out_lse), _stream(stream)),
           "mla_decode_attn")


NOALLOC_MAX_WORKSPACE = 96 << 20      # bytes of the library's own split workspace


def decode_attn_noalloc(dims: MLADims, q_abs, cache, kv_scale, page_table, max_pages: int,
                        max_len: int, seq_lens, seq_lens_host: Sequence[int], q_tokens: int,
                        num_splits: int, out_latent, out_lse, stream=None, _lens_cache=None):
    """mla_decode_attn with the split workspace in the library's device array."""
    lib = load_library()
    lens = _lens_cache if _lens_cache is not None else _lens_host(seq_lens_host)
    _check(lib.mla_decode_attn_noalloc(ctypes.byref(dims), _ptr(q_abs), _ptr(cache),
                                       _ptr(kv_scale), _ptr(page_table), int(max_pages),
                                       int(max_len), _ptr(seq_lens),
                                       ctypes.cast(lens, ctypes.c_void_p), len(seq_lens_host),
                                       int(q_tokens), int(num_splits), _ptr(out_latent),
                                       _ptr(out_lse), _stream(stream)),
           "mla_decode_attn_noalloc")


def absorb_append(dims: MLADims, q_nope, q_rope, w_uk, q_pos, q_abs, n_tokens: int,
                  new_c, new_kr, seq_idx, pos, page_table, batch: int, max_pages: int,
                  max_len: int, cache_rows: int, apply_rope: bool, cache, kv_scale,
                  n_rows: int, stream=None):
    """mla_absorb_q and mla_cache_append in one call (one launch on their fast paths)."""
    lib = load_library()
    _check(lib.mla_absorb_append(ctypes.byref(dims), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                 _ptr(q_pos), _ptr(q_abs), int(n_tokens), _ptr(new_c),
                                 _ptr(new_kr), _ptr(seq_idx), _ptr(pos), _ptr(page_table),
                                 int(batch), int(max_pages), int(max_len), int(cache_rows),
                                 int(bool(apply_rope)), _ptr(cache), _ptr(kv_scale),
                                 int(n_rows), _stream(stream)),
           "mla_absorb_append")


def check_page_table(dims: MLADims, page_table, max_pages: int, seq_lens, batch: int,
                     n_pages: int, result, stream=None):
    """Device range check of a page table; result: int32[4] on the device
    (out-of-range entries, first flat index or -1, its value, bad lengths)."""
    lib = load_library()
    _check(lib.mla_check_page_table(ctypes.byref(dims), _ptr(page_table), int(max_pages),
                                    _ptr(seq_lens), int(batch), int(n_pages), _ptr(result),
                                    _stream(stream)),
           "mla_check_page_table")


def up_proj_v(dims: MLADims, latent, w_uv, out, n_tokens: int, stream=None,
              out_dtype: Optional[int] = None):
    """out_dtype defaults to the dtype of ``out`` (float32 -> F32, else BF16)."""
    lib = load_library()
    if out_dtype is None:
        import torch
        out_dtype = F32 if (not isinstance(out, int) and out.dtype == torch.float32) else BF16
    _check(lib.mla_up_proj_v(ctypes.byref(dims), _ptr(latent), _ptr(w_uv), _ptr(out),
                             int(out_dtype), int(n_tokens), _stream(stream)),
           "mla_up_proj_v")


def out_proj_workspace_size(dims: MLADims, d_model: int, n_tokens: int, o_dtype: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.mla_out_proj_workspace_size(ctypes.byref(dims), int(d_model), int(n_tokens),
                                           int(o_dtype), ctypes.byref(out)),
           "mla_out_proj_workspace_size")
    return int(out.value)


def out_proj(dims: MLADims, o, w_o, d_model: int, u, n_tokens: int, workspace, ws_bytes: int,
             stream=None, o_dtype: Optional[int] = None, u_dtype: Optional[int] = None):
    """u = W^O [o_1; ...; o_{n_h}].  The dtypes default to those of the tensors
    (float32 -> F32, else BF16)."""
    lib = load_library()
    import torch

    def code(t):
        return F32 if (not isinstance(t, int) and t.dtype == torch.float32) else BF16
    o_dtype = code(o) if o_dtype is None else o_dtype
    u_dtype = code(u) if u_dtype is None else u_dtype
    _check(lib.mla_out_proj(ctypes.byref(dims), _ptr(o), int(o_dtype), _ptr(w_o), int(d_model),
                            _ptr(u), int(u_dtype), int(n_tokens), _ptr(workspace), int(ws_bytes),
                            _stream(stream)), "mla_out_proj")


def out_proj_pack(dims: MLADims, w_o, d_model: int, w_packed, stream=None):
    """W^O [d_model, n_h d_h] bf16 -> the panel layout of mla_out_proj_packed."""
    lib = load_library()
    _check(lib.mla_out_proj_pack(ctypes.byref(dims), _ptr(w_o), int(d_model), _ptr(w_packed),
                                 _stream(stream)), "mla_out_proj_pack")


def out_proj_packed(dims: MLADims, o, w_packed, d_model: int, u, n_tokens: int, workspace,
                    ws_bytes: int, stream=None, u_dtype: Optional[int] = None):
    """u = W^O [o_1; ...; o_{n_h}] with W^O in the panel layout (o bf16); u's
    dtype defaults to that of the tensor (float32 -> F32, else BF16)."""
    lib = load_library()
    import torch
    if u_dtype is None:
        u_dtype = F32 if (not isinstance(u, int) and u.dtype == torch.float32) else BF16
    _check(lib.mla_out_proj_packed(ctypes.byref(dims), _ptr(o), _ptr(w_packed), int(d_model),
                                   _ptr(u), int(u_dtype), int(n_tokens), _ptr(workspace),
                                   int(ws_bytes), _stream(stream)), "mla_out_proj_packed")


def kv_produce_workspace_size(dims: MLADims, d_model: int, n_rows: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.mla_kv_produce_workspace_size(ctypes.byref(dims), int(d_model), int(n_rows),
                                             ctypes.byref(out)), "mla_kv_produce_workspace_size")
    return int(out.value)


def kv_produce(dims: MLADims, h, d_model: int, w_dkv_kr, norm_gain, norm_eps: float, seq_idx,
               pos, page_table, batch: int, max_pages: int, max_len: int, cache_rows: int,
               apply_rope: bool, cache, kv_scale, n_rows: int, workspace, ws_bytes: int,
               stream=None):
    """Cache rows [RMSNorm(W^DKV h) | RoPE(W^KR h)] appended at (seq_idx, pos)."""
    lib = load_library()
    _check(lib.mla_kv_produce(ctypes.byref(dims), _ptr(h), int(d_model), _ptr(w_dkv_kr),
                              _ptr(norm_gain), float(norm_eps), _ptr(seq_idx), _ptr(pos),
                              _ptr(page_table), int(batch), int(max_pages), int(max_len),
                              int(cache_rows), int(bool(apply_rope)), _ptr(cache), _ptr(kv_scale),
                              int(n_rows), _ptr(workspace), int(ws_bytes), _stream(stream)),
           "mla_kv_produce")
