"""The C-ABI library loads, exports what include/mla.h declares, and rejects
invalid arguments with the documented status codes before any HIP call (so
these run without a GPU).  Also checks the host split planner through
mla_decode_workspace_size."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")
LIB = os.path.join(ROOT, "head_latent_attention_11_amd", "libmla.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmla.so not built")

OK, NULL, DIMS, DTYPE, ALIGN, SEQLEN, WS, UNSUP, LAUNCH, ARG = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
FAKE = 0x10000          # a 16-byte aligned non-null address, never dereferenced
MIS = 0x10008           # misaligned


@pytest.fixture(scope="module")
def mla():
    from head_latent_attention_11_amd import binding
    return binding.load_library(LIB), binding


def _declared():
    text = open(HEADER).read()
    return re.findall(r"^(?:int32_t|const char\*)\s+(mla_\w+)\s*\(", text, re.M)


def test_header_declarations_found():
    names = _declared()
    assert set(names) >= {"mla_absorb_q", "mla_cache_append", "mla_decode_workspace_size",
                          "mla_decode_attn", "mla_up_proj_v", "mla_status_string"}


def test_library_exports_every_declared_symbol(mla):
    lib, _ = mla
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings_and_version(mla):
    lib, b = mla
    for code in (OK, NULL, DIMS, DTYPE, ALIGN, SEQLEN, WS, UNSUP, LAUNCH, ARG, -1234):
        assert isinstance(b.status_string(code), str) and b.status_string(code)
    assert b.version() >= 10000


def _v2(b, n_heads=128, **kw):
    return b.MLADims.make(n_heads, 128, 512, 64, **kw)


def _decode(lib, b, dims, lens, T=1, q=FAKE, cache=FAKE, scale=None, pt=None, max_pages=0,
            max_len=8192, seq=FAKE, ws=None, wsb=0, out=FAKE, lse=FAKE, splits=0):
    arr = (ctypes.c_int32 * len(lens))(*lens)
    return lib.mla_decode_attn(ctypes.byref(dims), q, cache, scale, pt, max_pages, max_len, seq,
                               ctypes.cast(arr, ctypes.c_void_p), len(lens), T, splits, ws,
                               wsb, out, lse, None)


def test_decode_validation(mla):
    lib, b = mla
    d = _v2(b)
    assert _decode(lib, b, d, [100], q=None) == NULL
    assert _decode(lib, b, d, [100], out=None) == NULL
    assert _decode(lib, b, d, [100], q=MIS) == ALIGN
    assert _decode(lib, b, d, [0]) == SEQLEN                  # L_b = 0
    assert _decode(lib, b, d, [3], T=4) == SEQLEN             # T > L_b
    assert _decode(lib, b, d, [9000], max_len=8192) == SEQLEN  # beyond capacity
    assert _decode(lib, b, d, [100], T=0) == ARG
    assert _decode(lib, b, d, [100], splits=-1) == ARG
    assert _decode(lib, b, d, [4096] * 32) == WS              # needs a workspace
    assert _decode(lib, b, d, [4096] * 32, ws=FAKE, wsb=16) == WS
    fp8 = _v2(b, kv_dtype="fp8")
    assert _decode(lib, b, fp8, [100]) == NULL                # fp8 needs kv_scale
    bad = _v2(b, page_size=32)
    assert _decode(lib, b, bad, [100]) == DIMS
    bad = _v2(b, kv_dtype=7)
    assert _decode(lib, b, bad, [100]) == DTYPE
    bad = b.MLADims.make(128, 128, 512, 63)
    assert _decode(lib, b, bad, [100]) == DIMS                # odd RoPE dim
    bad = b.MLADims.make(128, 128, 513, 64)
    assert _decode(lib, b, bad, [100]) == DIMS
    bad = _v2(b, softmax_scale=-1.0)
    assert _decode(lib, b, bad, [100]) == ARG
    bad = _v2(b, precision=4)
    assert _decode(lib, b, bad, [100]) == ARG                 # unknown precision mode
    bad = _v2(b, precision=-1)
    assert _decode(lib, b, bad, [100]) == ARG
    # split operands need 128-head multiples and a bf16 cache
    assert _decode(lib, b, _v2(b, n_heads=16, precision="bf16x2"), [100]) == UNSUP
    assert _decode(lib, b, _v2(b, kv_dtype="fp8", precision="bf16x2"), [100],
                   scale=FAKE) == UNSUP
    # paged: capacity is max_pages * 64
    assert _decode(lib, b, d, [200], pt=FAKE, max_pages=3) == SEQLEN
    assert _decode(lib, b, d, [200], pt=FAKE, max_pages=0) == ARG
    assert lib.mla_decode_attn(None, FAKE, FAKE, None, None, 0, 10, FAKE, FAKE, 1, 1, 0,
                               None, 0, FAKE, FAKE, None) == NULL


def test_out_proj_validation(mla):
    lib, b = mla
    d = _v2(b)
    sz = ctypes.c_size_t(0)
    assert lib.mla_out_proj_workspace_size(ctypes.byref(d), 5120, 32, 1, ctypes.byref(sz)) == OK
    assert sz.value == 8 * 32 * 5120 * 4          # 8 K blocks of fp32 partials
    assert lib.mla_out_proj_workspace_size(ctypes.byref(d), 5120, 32, 0, ctypes.byref(sz)) == OK
    assert sz.value == 0                          # fp32 o: no matrix-core path, no workspace
    assert lib.mla_out_proj_workspace_size(ctypes.byref(d), 0, 32, 1, ctypes.byref(sz)) == ARG
    assert lib.mla_out_proj_workspace_size(ctypes.byref(d), 5120, 32, 2, ctypes.byref(sz)) == DTYPE
    op = lib.mla_out_proj
    assert op(ctypes.byref(d), None, 1, FAKE, 5120, FAKE, 0, 32, FAKE, 1 << 30, None) == NULL
    assert op(ctypes.byref(d), FAKE, 1, None, 5120, FAKE, 0, 32, FAKE, 1 << 30, None) == NULL
    assert op(ctypes.byref(d), FAKE, 2, FAKE, 5120, FAKE, 0, 32, FAKE, 1 << 30, None) == DTYPE
    assert op(ctypes.byref(d), FAKE, 1, FAKE, 5120, FAKE, 2, 32, FAKE, 1 << 30, None) == DTYPE
    assert op(ctypes.byref(d), FAKE, 1, FAKE, 5120, FAKE, 0, 0, FAKE, 1 << 30, None) == ARG
    assert op(ctypes.byref(d), FAKE, 1, FAKE, -1, FAKE, 0, 32, FAKE, 1 << 30, None) == ARG
    assert op(ctypes.byref(d), FAKE, 1, MIS, 5120, FAKE, 0, 32, FAKE, 1 << 30, None) == ALIGN
    assert op(ctypes.byref(d), FAKE, 1, FAKE, 5120, FAKE, 0, 32, None, 0, None) == WS
    assert op(ctypes.byref(d), FAKE, 1, FAKE, 5120, FAKE, 0, 32, FAKE, 1024, None) == WS


def test_out_proj_packed_validation(mla):
    lib, b = mla
    d = _v2(b)
    d32 = _v2(b, q_dtype="f32")
    W2 = FAKE + (1 << 30)               # a second buffer, clear of FAKE's 168 MB
    pk = lib.mla_out_proj_pack
    assert pk(ctypes.byref(d), None, 5120, W2, None) == NULL
    assert pk(ctypes.byref(d), FAKE, 5120, None, None) == NULL
    assert pk(ctypes.byref(d), FAKE, 0, W2, None) == ARG
    assert pk(ctypes.byref(d32), FAKE, 5120, W2, None) == DTYPE
    assert pk(ctypes.byref(d), FAKE, 5136, W2, None) == UNSUP       # d_model % 32 != 0
    assert pk(ctypes.byref(d), FAKE, 65536, W2, None) == UNSUP      # 2 GiB of W^O
    assert pk(ctypes.byref(d), MIS, 5120, W2, None) == ALIGN
    assert pk(ctypes.byref(d), FAKE, 5120, FAKE + 4096, None) == ARG  # overlapping
    op = lib.mla_out_proj_packed
    big = 1 << 30
    assert op(ctypes.byref(d), None, FAKE, 5120, FAKE, 0, 32, FAKE, big, None) == NULL
    assert op(ctypes.byref(d), FAKE, None, 5120, FAKE, 0, 32, FAKE, big, None) == NULL
    assert op(ctypes.byref(d), FAKE, FAKE, 5120, None, 0, 32, FAKE, big, None) == NULL
    assert op(ctypes.byref(d32), FAKE, FAKE, 5120, FAKE, 0, 32, FAKE, big, None) == DTYPE
    assert op(ctypes.byref(d), FAKE, FAKE, 5120, FAKE, 2, 32, FAKE, big, None) == DTYPE
    assert op(ctypes.byref(d), FAKE, FAKE, 5120, FAKE, 0, 0, FAKE, big, None) == ARG
    assert op(ctypes.byref(d), FAKE, FAKE, 0, FAKE, 0, 32, FAKE, big, None) == ARG
    assert op(ctypes.byref(d), FAKE, FAKE, 5136, FAKE, 0, 32, FAKE, big, None) == UNSUP
    assert op(ctypes.byref(d), FAKE, MIS, 5120, FAKE, 0, 32, FAKE, big, None) == ALIGN
    assert op(ctypes.byref(d), FAKE, FAKE, 5120, FAKE, 0, 32, None, 0, None) == WS
    assert op(ctypes.byref(d), FAKE, FAKE, 5120, FAKE, 0, 32, FAKE, 1024, None) == WS


def test_page_table_check_validation(mla):
    lib, b = mla
    d = _v2(b)
    chk = lib.mla_check_page_table
    assert chk(None, FAKE, 8, FAKE, 4, 100, FAKE, None) == NULL
    assert chk(ctypes.byref(d), None, 8, FAKE, 4, 100, FAKE, None) == NULL
    assert chk(ctypes.byref(d), FAKE, 8, None, 4, 100, FAKE, None) == NULL
    assert chk(ctypes.byref(d), FAKE, 8, FAKE, 4, 100, None, None) == NULL
    assert chk(ctypes.byref(d), FAKE, 0, FAKE, 4, 100, FAKE, None) == ARG
    assert chk(ctypes.byref(d), FAKE, 8, FAKE, 0, 100, FAKE, None) == ARG
    assert chk(ctypes.byref(d), FAKE, 8, FAKE, 4, 0, FAKE, None) == ARG
    assert chk(ctypes.byref(d), FAKE, 1 << 16, FAKE, 1 << 16, 100, FAKE, None) == ARG


def test_absorb_append_validation(mla):
    lib, b = mla
    d = _v2(b)
    aa = lib.mla_absorb_append

    def call(q_nope=FAKE, w_uk=FAKE, q_abs=FAKE, n_tok=4, new_c=FAKE, cache=FAKE, scale=None,
             n_rows=4, dims=d):
        return aa(ctypes.byref(dims) if dims is not None else None, q_nope, FAKE, w_uk, None,
                  q_abs, n_tok, new_c, FAKE, FAKE, FAKE, None, 2, 0, 64, 128, 0, cache, scale,
                  n_rows, None)
    assert call(dims=None) == NULL
    assert call(q_nope=None) == NULL
    assert call(q_abs=None) == NULL
    assert call(new_c=None) == NULL
    assert call(cache=None) == NULL
    assert call(n_tok=0) == ARG
    assert call(n_rows=0) == ARG
    assert call(q_abs=MIS) == ALIGN
    assert call(cache=MIS) == ALIGN
    assert call(scale=FAKE) == ARG                     # scales only with an fp8 cache
    d8 = _v2(b, kv_dtype="fp8")
    assert call(dims=d8) == NULL                        # fp8 cache without scales


def test_kv_produce_validation(mla):
    lib, b = mla
    d = _v2(b)
    sz = ctypes.c_size_t(0)
    assert lib.mla_kv_produce_workspace_size(ctypes.byref(d), 5120, 32, ctypes.byref(sz)) == OK
    assert sz.value == 20 * 32 * 576 * 4           # partial sums of 20 K blocks of 256
    assert lib.mla_kv_produce_workspace_size(ctypes.byref(d), 0, 32, ctypes.byref(sz)) == ARG
    kp = lib.mla_kv_produce

    def call(h=FAKE, w=FAKE, gain=None, eps=1e-6, seq=FAKE, pos=FAKE, pt=None, batch=4,
             max_pages=0, max_len=128, rows=512, rope=1, cache=FAKE, scale=None, n=8,
             d_model=5120, ws=FAKE, wsb=1 << 30, dims=d):
        return kp(ctypes.byref(dims), h, d_model, w, gain, eps, seq, pos, pt, batch, max_pages,
                  max_len, rows, rope, cache, scale, n, ws, wsb, None)
    assert call(h=None) == NULL
    assert call(w=None) == NULL
    assert call(seq=None) == NULL
    assert call(cache=None) == NULL
    assert call(dims=_v2(b, kv_dtype="fp8")) == NULL          # fp8 needs kv_scale
    assert call(scale=FAKE) == ARG                             # a scale without fp8
    assert call(n=0) == ARG
    assert call(rope=2) == ARG
    assert call(d_model=0) == ARG
    assert call(eps=-1.0) == ARG
    assert call(eps=float("inf")) == ARG
    assert call(max_len=200) == ARG                            # batch * max_len > cache rows
    assert call(h=MIS) == ALIGN
    assert call(gain=MIS) == ALIGN
    assert call(ws=None, wsb=0) == WS
    assert call(wsb=64) == WS


def test_absorb_append_upproj_validation(mla):
    lib, b = mla
    d = _v2(b)
    assert lib.mla_absorb_q(ctypes.byref(d), None, FAKE, FAKE, None, FAKE, 4, None) == NULL
    assert lib.mla_absorb_q(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, 0, None) == ARG
    assert lib.mla_absorb_q(ctypes.byref(d), FAKE, FAKE, MIS, None, FAKE, 4, None) == ALIGN
    assert lib.mla_up_proj_v(ctypes.byref(d), FAKE, None, FAKE, 0, 4, None) == NULL
    assert lib.mla_up_proj_v(ctypes.byref(d), FAKE, FAKE, MIS, 0, 4, None) == ALIGN
    assert lib.mla_up_proj_v(ctypes.byref(d), FAKE, FAKE, FAKE, 2, 4, None) == DTYPE
    assert lib.mla_up_proj_v(ctypes.byref(d), FAKE, FAKE, FAKE, 0, -1, None) == ARG
    ap = lib.mla_cache_append
    assert ap(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 2, 0, 64, 128, 0, FAKE, None,
              0, None) == ARG                                  # n_rows = 0
    assert ap(ctypes.byref(d), FAKE, FAKE, None, FAKE, None, 2, 0, 64, 128, 0, FAKE, None,
              8, None) == NULL
    assert ap(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 2, 0, 64, 100, 0, FAKE, None,
              8, None) == ARG                                  # B*max_len > rows
    assert ap(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 2, 0, 64, 128, 0, FAKE, FAKE,
              8, None) == ARG                                  # scale on a bf16 cache
    fp8 = _v2(b, kv_dtype="fp8")
    assert ap(ctypes.byref(fp8), FAKE, FAKE, FAKE, FAKE, None, 2, 0, 64, 128, 0, FAKE, None,
              8, None) == NULL                                 # fp8 needs the scale array
    assert ap(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 2, 0, 64, 128, 2, FAKE, None,
              8, None) == ARG                                  # apply_rope not 0/1
    assert ap(ctypes.byref(d), MIS, FAKE, FAKE, FAKE, None, 2, 0, 64, 128, 0, FAKE, None,
              8, None) == ALIGN


def test_yarn_settings_validation(mla):
    lib, b = mla
    assert _ws(lib, _v2(b, yarn_factor=40.0), [4096])[0] == OK
    assert _ws(lib, _v2(b, yarn_factor=1.0, yarn_alpha=0.0), [4096])[0] == OK   # off: unchecked
    for bad in (dict(yarn_factor=-1.0), dict(yarn_factor=float("nan")),
                dict(yarn_factor=40.0, yarn_alpha=0.0),
                dict(yarn_factor=40.0, yarn_beta=0.5),                  # beta <= alpha
                dict(yarn_factor=40.0, yarn_orig_len=0),
                dict(yarn_factor=40.0, yarn_coef=-0.1),
                dict(yarn_factor=40.0, yarn_beta=float("inf"))):
        assert _ws(lib, _v2(b, **bad), [4096])[0] == ARG, bad


def _ws(lib, dims, lens, T=1, splits=0):
    arr = (ctypes.c_int32 * len(lens))(*lens)
    out = ctypes.c_size_t(0)
    st = lib.mla_decode_workspace_size(ctypes.byref(dims), ctypes.cast(arr, ctypes.c_void_p),
                                       len(lens), T, splits, ctypes.byref(out))
    return st, out.value


def test_split_planner_sizes(mla):
    lib, b = mla
    d = _v2(b, precision="bf16")          # bf16 operands only: bf16 partials
    rows, dc = 128, 512
    # 32 x 4096 tokens, 1 row block of 128 rows: chunk 512 -> 8 splits each
    st, n = _ws(lib, d, [4096] * 32)
    assert st == OK and n == 256 * rows * 4 + 256 * rows * dc * 2   # fp32 LSE + bf16 partials
    # 64 x 8192, T = 4 (4 row blocks): chunk 8192 -> no split, no workspace
    st, n = _ws(lib, _v2(b, kv_dtype="fp8"), [8192] * 64, T=4)
    assert st == OK and n == 0
    # explicit 64 splits of 131072 tokens: 4 * 64 items
    st, n = _ws(lib, d, [131072] * 4, splits=64)
    assert st == OK and n == 256 * rows * 4 + 256 * rows * dc * 2
    # 16 heads (one block of 16 rows): 32 x 4096 tokens fill 256 items of 512
    st, n = _ws(lib, _v2(b, n_heads=16), [4096] * 32)
    assert st == OK and n == 256 * 16 * 4 + 256 * 16 * dc * 2
    # 48 heads: three blocks of 16 rows, 86 items wanted -> chunk 1536, 3 splits
    st, n = _ws(lib, _v2(b, n_heads=48), [4096] * 32)
    assert st == OK and n == 96 * 48 * 4 + 96 * 48 * dc * 2
    # 16 heads x T = 4 on an fp8 cache: two blocks of 32 rows, 128 items
    # wanted -> chunk 4096, 2 splits each; 64 x 8192 with T = 1: chunk 2048,
    # 4 splits each (the V2-Lite benchmark workload)
    st, n = _ws(lib, _v2(b, n_heads=16, kv_dtype="fp8"), [8192] * 64, T=4)
    assert st == OK and n == 128 * 64 * 4 + 128 * 64 * dc * 2
    st, n = _ws(lib, _v2(b, n_heads=16), [8192] * 64)
    assert st == OK and n == 256 * 16 * 4 + 256 * 16 * dc * 2
    # head counts that are no multiple of 16 (general path, one workgroup per
    # row): 8 rows want 32 items -> chunk 4096, no split; with 8 splits the
    # partials are fp32
    st, n = _ws(lib, _v2(b, n_heads=8), [4096] * 32)
    assert st == OK and n == 0
    st, n = _ws(lib, _v2(b, n_heads=8), [4096] * 32, splits=8)
    assert st == OK and n == 256 * 8 * 4 + 256 * 8 * dc * 4
    # fp32 precision mode: same items, fp32 partials
    st, n = _ws(lib, _v2(b, precision=1), [131072] * 4, splits=64)
    assert st == OK and n == 256 * rows * 4 + 256 * rows * dc * 4
    # a short sequence is never split below 256 tokens
    st, n = _ws(lib, d, [200])
    assert st == OK and n == 0
    st, _ = _ws(lib, d, [5], T=6)
    assert st == SEQLEN


def test_split_planner_sizes_with_split_operands(mla):
    """Precision AUTO (128 heads, bf16 cache): partial slots of fp32 size and
    one flag per (item, 128-row block), each part 256-byte aligned; BF16X2:
    fp32 partials, no flags; the items are planned as for 128-row blocks."""
    lib, b = mla
    rows, dc = 128, 512
    auto = _v2(b)
    assert auto.precision == 0
    st, n = _ws(lib, auto, [4096] * 32)                        # 256 items of 512 tokens
    assert st == OK and n == 256 * rows * 4 + 256 * rows * dc * 4 + 1024
    st, n = _ws(lib, auto, [131072] * 4, splits=64)
    assert st == OK and n == 256 * rows * 4 + 256 * rows * dc * 4 + 1024
    st, n = _ws(lib, auto, [8192] * 64, T=4)                   # unsplit: flags only
    assert st == OK and n == 64 * 4 * 4
    st, n = _ws(lib, auto, [200])                              # one flag, 256-byte aligned
    assert st == OK and n == 256
    st, n = _ws(lib, _v2(b, kv_dtype="fp8"), [8192] * 64, T=4)  # fp8 cache: no escalation
    assert st == OK and n == 0
    x2 = _v2(b, precision="bf16x2")
    st, n = _ws(lib, x2, [4096] * 32)
    assert st == OK and n == 256 * rows * 4 + 256 * rows * dc * 4
    st, n = _ws(lib, x2, [200])
    assert st == OK and n == 0
    st, _ = _ws(lib, _v2(b, n_heads=64, precision="bf16x2"), [4096])
    assert st == UNSUP


def test_dims_struct_layout_matches_header(tmp_path):
    """The binding's mirror of mla_dims_t has the header's size and field
    offsets: a C program built from include/mla.h prints them."""
    import shutil
    import subprocess
    from head_latent_attention_11_amd import binding
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = [f[0] for f in binding.MLADims._fields_]
    src = tmp_path / "dims.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "mla.h"\n'
        "int main(void) {\n"
        '  printf("%zu\\n", sizeof(mla_dims_t));\n'
        + "".join(f'  printf("%zu\\n", offsetof(mla_dims_t, {n}));\n' for n in names)
        + "  return 0;\n}\n")
    exe = tmp_path / "dims"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(binding.MLADims)
    assert out[1:] == [getattr(binding.MLADims, n).offset for n in names]


def test_noalloc_rejects_plans_beyond_its_array(mla):
    """mla_decode_attn_noalloc checks the plan's workspace against its
    96 MiB device array on the host, before any HIP call."""
    lib, b = mla
    d = _v2(b)
    lens = [65536] * 64
    arr = (ctypes.c_int32 * len(lens))(*lens)
    need = b.decode_workspace_size(d, lens, 1, 64)
    assert need > b.NOALLOC_MAX_WORKSPACE
    assert lib.mla_decode_attn_noalloc(ctypes.byref(d), FAKE, FAKE, None, None, 0, 65536, FAKE,
                                       ctypes.cast(arr, ctypes.c_void_p), len(lens), 1, 64,
                                       FAKE, FAKE, None) == WS
    assert lib.mla_decode_attn_noalloc(ctypes.byref(d), None, FAKE, None, None, 0, 65536, FAKE,
                                       ctypes.cast(arr, ctypes.c_void_p), len(lens), 1, 64,
                                       FAKE, FAKE, None) == NULL


def test_six_bit_cache_validation(mla):
    """The 6-bit cache: 128-row attention blocks only, rows of 576 elements,
    no per-row scale array."""
    lib, b = mla
    fp6 = _v2(b, kv_dtype="fp6")
    assert fp6.kv_dtype == 3
    st, n = _ws(lib, fp6, [8192] * 64, T=4)                  # unsplit, no flags
    assert st == OK and n == 0
    assert _decode(lib, b, _v2(b, n_heads=16, kv_dtype="fp6"), [100]) == UNSUP
    assert _decode(lib, b, _v2(b, kv_dtype="fp6", precision="fp32"), [100]) == UNSUP
    assert _decode(lib, b, _v2(b, kv_dtype="fp6", precision="bf16x2"), [100]) == UNSUP
    one = (ctypes.c_int32 * 1)(0)
    ap = lambda d, scale: lib.mla_cache_append(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 1, 0,
                                               64, 64, 0, FAKE, scale, 1, None)
    assert ap(fp6, FAKE) == ARG                                # no scale array
    assert ap(b.MLADims.make(128, 128, 256, 64, kv_dtype="fp6"), None) == UNSUP   # D != 576
