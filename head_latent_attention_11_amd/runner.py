"""Device buffers and one decode step through the C ABI.

``DecodeBuffers`` uploads a generated workload (numpy arrays from
``mla_inputs.generate``) into torch-allocated GPU memory, fills the latent
cache with ``mla_cache_append`` (so the cache bytes are written by the
library's own append kernel), and runs the decode step

    mla_absorb_append (mla_absorb_q + mla_cache_append in one call)
    -> mla_decode_attn (split-KV + combine) -> mla_up_proj_v

on the current torch stream (the step appends its B*T new rows before the
attention call; absorb() and append() run the two separately).  No
arithmetic of the method happens here.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import binding as B

_TORCH_STORE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(arr: np.ndarray, kind: str, device) -> torch.Tensor:
    """Upload a generator array: 'bf16' arrays are uint16 bit patterns."""
    if kind == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    if kind == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    if kind == "i32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).to(device)
    raise ValueError(kind)


class DecodeBuffers:
    def __init__(self, w, gen: Dict[str, np.ndarray], device="cuda",
                 num_splits: Optional[int] = None, poison: bool = True,
                 cache_replicas: int = 1, precision: str = "auto",
                 weight_replicas: int = 1):
        self.w = w
        self.device = torch.device(device)
        dev = self.device
        self.precision = precision
        self.dims = B.MLADims.from_workload(w, precision)
        qk = "f32" if w.q_dtype == "f32" else "bf16"
        self.w_uk = to_device(gen["w_uk"], qk, dev)
        self.w_uv = to_device(gen["w_uv"], qk, dev)
        # copies of W^UK / W^UV used round-robin with the cache replicas, so
        # that a step reads its weights from HBM as a layer of a whole model
        # would, not from the memory-side cache
        self.w_uks = [self.w_uk] + [self.w_uk.clone() for _ in range(max(1, weight_replicas) - 1)]
        self.w_uvs = [self.w_uv] + [self.w_uv.clone() for _ in range(max(1, weight_replicas) - 1)]
        self.q_nope = to_device(gen["q_nope"], qk, dev)
        self.q_rope = to_device(gen["q_rope"], qk, dev)
        self.q_pos = to_device(gen["q_pos"], "i32", dev) if w.rope else None
        self.seq_lens_host = [int(x) for x in gen["seq_lens"]]
        self.seq_lens = to_device(gen["seq_lens"], "i32", dev)
        self.batch = w.batch
        self.T = w.q_tokens
        self.n_tok = w.batch * w.q_tokens
        self.num_splits = w.num_splits if num_splits is None else num_splits
        D = w.d_latent + w.d_rope

        # ---- cache storage
        if w.layout == "paged":
            self.page_table = to_device(gen["page_table"], "i32", dev)
            self.max_pages = int(gen["page_table"].shape[1])
            self.max_len = 0
            self.cache_rows = int(gen["num_pages"]) * w.page_size
        else:
            self.page_table = None
            self.max_pages = 0
            self.max_len = int(max(self.seq_lens_host))
            self.cache_rows = w.batch * self.max_len
        self.caches = []
        self.scales = []
        for _ in range(max(1, cache_replicas)):
            if w.kv_dtype == "fp8":
                cache = torch.empty((self.cache_rows, D), dtype=torch.uint8, device=dev)
                scale = torch.empty((self.cache_rows,), dtype=torch.float32, device=dev)
                if poison:
                    cache.fill_(0x7F)                       # E4M3 NaN
                    scale.fill_(float("nan"))
            elif w.kv_dtype == "fp6":
                cache = torch.empty((self.cache_rows, B.FP6_ROW_BYTES), dtype=torch.uint8,
                                    device=dev)
                scale = None
                if poison:
                    cache.fill_(0xFF)                       # exponent byte 255: infinite scale
            else:
                cache = torch.empty((self.cache_rows, D), dtype=_TORCH_STORE[w.kv_dtype], device=dev)
                scale = None
                if poison:
                    cache.fill_(float("nan"))
            self.caches.append(cache)
            self.scales.append(scale)
        self.cache, self.kv_scale = self.caches[0], self.scales[0]

        # ---- fill the cache with the library's append kernel (bulk prefill)
        src = "f32" if w.kv_dtype == "f32" else "bf16"
        new_c = to_device(gen["c_kv"], src, dev)
        new_kr = to_device(gen["k_r"], src, dev)
        seq_idx = to_device(gen["row_seq"], "i32", dev)
        pos = to_device(gen["row_pos"], "i32", dev)
        for cache, scale in zip(self.caches, self.scales):
            B.cache_append(self.dims, new_c, new_kr, seq_idx, pos, self.page_table,
                           w.batch, self.max_pages, self.max_len, self.cache_rows,
                           w.rope, cache, scale, new_c.shape[0])
        # ---- the step's own B*T new rows (positions L_b - T .. L_b - 1 of each
        # sequence), appended again by every step: the append of a decode
        # step.  Writing the same row twice stores the same bytes, so a step
        # leaves the prefilled cache as it is.
        offs = np.asarray(gen["row_offsets"], dtype=np.int64)
        lens = np.asarray(gen["seq_lens"], dtype=np.int64)
        rows = np.concatenate([offs[b] + np.arange(lens[b] - self.T, lens[b])
                               for b in range(w.batch)])
        self.new_c = new_c[torch.from_numpy(rows).to(dev)].contiguous()
        self.new_kr = new_kr[torch.from_numpy(rows).to(dev)].contiguous()
        self.new_seq = seq_idx[torch.from_numpy(rows).to(dev)].contiguous()
        self.new_pos = pos[torch.from_numpy(rows).to(dev)].contiguous()
        del new_c, new_kr, seq_idx, pos

        # ---- outputs and workspace
        qabs_dtype = torch.float32 if self.dims.qabs_is_f32() else self.w_uk.dtype
        qshape = ((self.n_tok, w.n_heads, 2, D) if self.dims.qabs_pairs()
                  else (self.n_tok, w.n_heads, D))
        self.q_abs = torch.empty(qshape, dtype=qabs_dtype, device=dev)
        self.latent = torch.empty((self.n_tok, w.n_heads, w.d_latent), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.n_tok, w.n_heads), dtype=torch.float32, device=dev)
        # o is written in fp32: the parity gates are absolute (max-abs) and the
        # long-context outliers give |o| ~ 20, where bf16 rounding alone is ~0.04
        self.o = torch.empty((self.n_tok, w.n_heads, w.d_head), dtype=torch.float32, device=dev)
        if poison:
            for t in (self.q_abs, self.latent, self.lse, self.o):
                t.fill_(float("nan"))
        self.ws_bytes = B.decode_workspace_size(self.dims, self.seq_lens_host, self.T,
                                                self.num_splits)
        self.workspace = (torch.empty((self.ws_bytes + 15) // 16 * 4, dtype=torch.float32,
                                      device=dev) if self.ws_bytes else None)
        if self.workspace is not None and poison:
            self.workspace.fill_(float("nan"))
        self._lens_c = B._lens_host(self.seq_lens_host)

    # ----------------------------------------------------------- the step
    def absorb(self, stream=None, replica: int = 0):
        B.absorb_q(self.dims, self.q_nope, self.q_rope, self.w_uks[replica % len(self.w_uks)],
                   self.q_pos, self.q_abs, self.n_tok, stream)

    def append(self, stream=None, replica: int = 0):
        B.cache_append(self.dims, self.new_c, self.new_kr, self.new_seq, self.new_pos,
                       self.page_table, self.batch, self.max_pages, self.max_len,
                       self.cache_rows, self.w.rope, self.caches[replica],
                       self.scales[replica], self.n_tok, stream)

    def attend(self, replica: int = 0, stream=None, num_splits: Optional[int] = None):
        ns = self.num_splits if num_splits is None else num_splits
        ws, wsb = self.workspace, self.ws_bytes
        if ns != self.num_splits:
            wsb = B.decode_workspace_size(self.dims, self.seq_lens_host, self.T, ns)
            ws = torch.empty((wsb + 15) // 16 * 4, dtype=torch.float32,
                             device=self.device) if wsb else None
        B.decode_attn(self.dims, self.q_abs, self.caches[replica], self.scales[replica],
                      self.page_table, self.max_pages, self.max_len, self.seq_lens,
                      self.seq_lens_host, self.T, ns, ws, wsb, self.latent, self.lse,
                      stream, _lens_cache=self._lens_c)

    def up_proj(self, stream=None, replica: int = 0):
        B.up_proj_v(self.dims, self.latent, self.w_uvs[replica % len(self.w_uvs)], self.o,
                    self.n_tok, stream)

    def absorb_append(self, stream=None, replica: int = 0):
        """absorb() and append() as one library call (mla_absorb_append)."""
        B.absorb_append(self.dims, self.q_nope, self.q_rope, self.w_uks[replica % len(self.w_uks)],
                        self.q_pos, self.q_abs, self.n_tok, self.new_c, self.new_kr,
                        self.new_seq, self.new_pos, self.page_table, self.batch,
                        self.max_pages, self.max_len, self.cache_rows, self.w.rope,
                        self.caches[replica], self.scales[replica], self.n_tok, stream)

    def step(self, replica: int = 0, stream=None):
        self.absorb_append(stream, replica)
        self.attend(replica, stream)
        self.up_proj(stream, replica)
