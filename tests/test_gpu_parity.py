"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases compare every output element with the oracle; the full-size
workloads (in the launch configuration the benchmark times) compare sampled
(sequence, head) rows that the oracle computes one by one.  NaN poisoning:
the cache (including unused page slots and page tails), the outputs and the
split workspace are filled with NaN before the step, so any read of an
unwritten slot or a masked tile entering the PV product shows up as NaN.
"""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_support import (LSE_ABS, MAX_ABS_BF16, REL_L2_BF16, REL_L2_FP8, REL_L2_FP32_TARGET,
                         check, rel_l2, sample_mask, say, to_np)
from mla_inputs import WORKLOADS, generate, small_variant
from oracle import formats
from oracle import mla as omla
from oracle.rope import yarn_theta

pytestmark = pytest.mark.gpu

V2 = WORKLOADS["v2_b32_l4k_bf16"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_11_amd import binding
    binding.load_library()
    torch.cuda.set_device(0)


def _buffers(w, gen, **kw):
    from head_latent_attention_11_amd.runner import DecodeBuffers
    return DecodeBuffers(w, gen, device="cuda", **kw)


def _gates(w):
    # quantised caches (fp8, 6-bit): the rel-L2 gate of the fp8 cache, against
    # the oracle on the dequantised cache
    return (REL_L2_FP8, None) if w.kv_dtype in ("fp8", "fp6") else (REL_L2_BF16, MAX_ABS_BF16)


def _run_compare(w, gen=None, seqs=None, heads=None, num_splits=None, precision="auto",
                 max_abs=True, top_abs=0):
    """Step on the GPU, then compare the sampled rows (seqs x heads, all rows
    when None) with the oracle.  top_abs > 0 also compares the top_abs
    (query token, head) rows with the largest |o| of the GPU output (where an
    error in the score of a dominant token shows most), each recomputed by
    the oracle."""
    say(f"case {w.name}: B={w.batch} T={w.q_tokens} kv={w.kv_dtype} layout={w.layout} "
        f"splits={w.num_splits if num_splits is None else num_splits} precision={precision} "
        f"seqs={seqs} heads={heads} top_abs={top_abs}")
    gen = generate(w) if gen is None else gen
    buf = _buffers(w, gen, num_splits=num_splits, precision=precision)
    buf.step()
    torch.cuda.synchronize()
    o, lat, lse = to_np(buf.o), to_np(buf.latent), to_np(buf.lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lat)), "NaN/Inf in GPU output"
    assert np.all(np.isfinite(lse))
    ref = omla.decode_workload(gen, w, seqs=seqs, heads=heads)
    mask = sample_mask((w.batch * w.q_tokens, w.n_heads),
                       range(w.batch) if seqs is None else seqs,
                       range(w.n_heads) if heads is None else heads, w.q_tokens)
    if top_abs > 0:
        amax = np.abs(o).max(axis=2)
        order = np.argsort(amax, axis=None)[::-1][:top_abs]
        for flat in order:
            n, i = divmod(int(flat), w.n_heads)
            b = n // w.q_tokens
            say(f"  largest |o|: token {n} (seq {b}) head {i}: {amax[n, i]:.3f}")
            r1 = omla.decode_workload(gen, w, seqs=[b], heads=[i])
            for k in ("o", "latent", "lse"):
                ref[k][n, i] = r1[k][n, i]
            mask[n, i] = True
    rel, mabs = _gates(w)
    if not max_abs:
        mabs = None
    check("o", o[mask], ref["o"][mask], rel, mabs)
    check("latent", lat[mask], ref["latent"][mask], rel, mabs)
    dl = float(np.max(np.abs(lse[mask] - ref["lse"][mask])))
    say(f"  lse: max-abs {dl:.3e}" + (f" (gate {LSE_ABS:.0e})" if max_abs else ""))
    if max_abs:                    # LSE error is the score error: same cause as max-abs
        assert dl <= LSE_ABS
    if w.q_dtype == "f32" and w.kv_dtype == "f32":
        check("o (fp32 target)", o[mask], ref["o"][mask], REL_L2_FP32_TARGET)
    return buf, gen, ref


# ----------------------------------------------------------- small cases
# Every case runs in the default precision mode (AUTO): on the workloads with
# cache rows scaled by 8 the bf16 kernel hands its work items to the
# split-operand kernel, and both gates hold there.
SMALL = [
    WORKLOADS["tiny_fp32"],
    small_variant(V2, name="v2_ragged_auto", batch=4, kv_len=0, lengths=(1, 33, 700, 64)),
    small_variant(V2, name="v2_ragged_split5", batch=4, kv_len=0, lengths=(1, 33, 700, 64),
                  num_splits=5),
    small_variant(V2, name="v2_paged", batch=5, kv_len=0, lengths=(40, 900, 64, 65, 333),
                  layout="paged"),
    small_variant(V2, name="v2_outliers_split7", batch=2, kv_len=0, lengths=(3000, 2900),
                  num_splits=7, outlier_frac=0.01, outlier_scale=8.0),
    # more than 16 splits in one sequence (the one-workgroup-per-row combine),
    # uneven split counts across sequences, an unsplit sequence
    small_variant(V2, name="v2_ragged_split40", batch=3, kv_len=0, lengths=(2600, 64, 1300),
                  num_splits=40),
    small_variant(V2, name="bf16_t4", batch=2, q_tokens=4, kv_len=0, lengths=(129, 64)),
    small_variant(V2, name="fp8_t4", batch=4, q_tokens=4, kv_len=0, lengths=(300, 77, 4, 130),
                  kv_dtype="fp8"),
    small_variant(V2, name="fp8_t4_split3", batch=4, q_tokens=4, kv_len=0,
                  lengths=(300, 77, 4, 130), kv_dtype="fp8", num_splits=3),
    small_variant(V2, name="fp8_t1_paged", batch=2, kv_len=0, lengths=(100, 520),
                  kv_dtype="fp8", layout="paged"),
    # 128-row blocks holding several query tokens (32 or 64 heads): the waves
    # of a workgroup reach their visibility limits at different tiles, so they
    # switch from the fused steady-state step to the split step at different
    # steps between the same barriers
    small_variant(V2, name="fp8_n32_t4", batch=4, n_heads=32, q_tokens=4, kv_len=0,
                  lengths=(300, 97, 4, 1000), kv_dtype="fp8"),
    small_variant(V2, name="fp8_n64_t2_split3", batch=3, n_heads=64, q_tokens=2, kv_len=0,
                  lengths=(700, 130, 2), kv_dtype="fp8", num_splits=3),
    # lengths on tile boundaries: every tile of the item fully visible, and
    # one token past a boundary
    small_variant(V2, name="fp8_t1_tile_edges", batch=3, kv_len=0, lengths=(512, 65, 32),
                  kv_dtype="fp8"),
    # head counts with no multiple of 128 rows: the 16/32/64-row kernel
    small_variant(V2, name="lite_n16_ragged", batch=4, n_heads=16, kv_len=0,
                  lengths=(1, 33, 700, 64)),
    small_variant(V2, name="lite_n16_split5", batch=4, n_heads=16, kv_len=0,
                  lengths=(1, 33, 700, 64), num_splits=5),
    small_variant(V2, name="lite_n16_paged", batch=5, n_heads=16, kv_len=0,
                  lengths=(40, 900, 64, 65, 333), layout="paged"),
    small_variant(V2, name="lite_n16_t2", batch=3, n_heads=16, q_tokens=2, kv_len=0,
                  lengths=(129, 64, 3)),
    small_variant(V2, name="lite_n16_t4_split3", batch=4, n_heads=16, q_tokens=4, kv_len=0,
                  lengths=(300, 77, 4, 130), num_splits=3),
    small_variant(V2, name="lite_n16_t4_paged", batch=2, n_heads=16, q_tokens=4, kv_len=0,
                  lengths=(520, 100), layout="paged"),
    small_variant(V2, name="n48_t1", batch=3, n_heads=48, kv_len=0, lengths=(700, 64, 1)),
    small_variant(V2, name="n64_t1_split40", batch=3, n_heads=64, kv_len=0,
                  lengths=(2600, 64, 1300), num_splits=40),
    small_variant(V2, name="n96_t2", batch=2, n_heads=96, q_tokens=2, kv_len=0,
                  lengths=(333, 65)),
    small_variant(V2, name="lite_n16_rope", batch=2, n_heads=16, kv_len=0,
                  lengths=(70, 129), rope=True),
    small_variant(V2, name="general_n8_bf16", batch=2, n_heads=8, kv_len=0,
                  lengths=(50, 300)),
    small_variant(V2, name="lite_n16_fp8_rope", batch=2, n_heads=16, kv_len=0,
                  lengths=(70, 129), kv_dtype="fp8", rope=True),
    small_variant(V2, name="lite_n16_fp8_split5", batch=4, n_heads=16, kv_len=0,
                  lengths=(1, 33, 700, 64), kv_dtype="fp8", num_splits=5),
    small_variant(V2, name="lite_n16_fp8_t4_paged", batch=3, n_heads=16, q_tokens=4,
                  kv_len=0, lengths=(520, 100, 4), kv_dtype="fp8", layout="paged"),
    small_variant(V2, name="n32_fp8_t1", batch=3, n_heads=32, kv_len=0, lengths=(333, 65, 1000),
                  kv_dtype="fp8"),
    # the 6-bit cache (E2M3 codes, one power of two per 32 elements)
    small_variant(V2, name="fp6_t1_ragged", batch=4, kv_len=0, lengths=(1, 33, 700, 64),
                  kv_dtype="fp6"),
    small_variant(V2, name="fp6_t4_split3", batch=4, q_tokens=4, kv_len=0,
                  lengths=(300, 77, 4, 130), kv_dtype="fp6", num_splits=3),
    small_variant(V2, name="fp6_t1_paged", batch=3, kv_len=0, lengths=(100, 520, 31),
                  kv_dtype="fp6", layout="paged"),
    small_variant(V2, name="fp6_t2_rope_yarn", batch=2, q_tokens=2, kv_len=0,
                  lengths=(4600, 900), kv_dtype="fp6", rope=True, yarn_factor=40.0),
    small_variant(V2, name="general_n8_fp8", batch=2, n_heads=8, kv_len=0, lengths=(50, 300),
                  kv_dtype="fp8"),
    small_variant(WORKLOADS["tiny_fp32"], name="tiny_fp32_bf16cache", kv_dtype="bf16",
                  batch=2, kv_len=0, lengths=(64, 300), num_splits=2),
    small_variant(WORKLOADS["tiny_fp32"], name="tiny_fp32_yarn", yarn_factor=8.0,
                  yarn_orig_len=16, yarn_beta=8.0),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_decode_parity_small(w):
    _run_compare(w)


# Context extension (YaRN) of the RoPE parts, rotated by the library (query
# absorption and cache append) at positions past the 4K context, and the
# logit factor (c ln s + 1)^2 in the attention; sampled heads.
YARN = [
    (small_variant(V2, name="v2_yarn_rope", batch=3, kv_len=0, lengths=(5000, 700, 4500),
                   rope=True, yarn_factor=40.0), [0, 77, 127]),
    (small_variant(V2, name="lite_yarn_rope", batch=3, n_heads=16, kv_len=0,
                   lengths=(5000, 700, 4500), rope=True, yarn_factor=40.0, yarn_coef=0.1),
     [0, 9, 15]),
    (small_variant(V2, name="v2_yarn_fp8_t4", batch=2, q_tokens=4, kv_len=0,
                   lengths=(4600, 900), rope=True, yarn_factor=40.0, kv_dtype="fp8"),
     [0, 64, 127]),
    (small_variant(V2, name="lite_yarn_fp8_paged", batch=2, n_heads=16, kv_len=0,
                   lengths=(4600, 900), rope=True, yarn_factor=40.0, kv_dtype="fp8",
                   layout="paged"),
     [0, 15]),
]


@pytest.mark.parametrize("w,heads", YARN, ids=[c[0].name for c in YARN])
def test_decode_parity_yarn(w, heads):
    _run_compare(w, heads=heads)


def test_small_rows_long_paged_item():
    """One unsplit item of 9000 tokens in 64-token pages (141 pages: more
    than the 128 page ids the 16-row kernel keeps in registers, so it reads
    the page table per tile)."""
    w = small_variant(V2, name="lite_long_item", batch=2, n_heads=16, kv_len=0,
                      lengths=(9000, 300), layout="paged", num_splits=1)
    _run_compare(w, heads=[0, 5, 15])


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_long_paged_item_128_rows(kv):
    """The same on the 128-row kernels: an unsplit 9000-token paged item
    reads its page ids per tile with scalar loads, between the step
    sequences (fp8: also between the fused steady-state steps)."""
    w = small_variant(V2, name=f"long_item_{kv}", batch=2, kv_len=0, lengths=(9000, 300),
                      layout="paged", num_splits=1, kv_dtype=kv)
    _run_compare(w, heads=[0, 37, 127])


def test_small_rows_items_located_on_device():
    """More work items than the host's item table holds, lengths not all
    equal: the 16-row kernel locates each item from the lengths itself."""
    lengths = tuple(200 + (37 * i) % 1500 for i in range(40))
    w = small_variant(V2, name="lite_many_items", batch=40, n_heads=16, kv_len=0,
                      lengths=lengths, num_splits=40, layout="paged")
    n_items = sum(-(-L // (-(-(-(-L // 40)) // 64) * 64)) for L in lengths)
    assert n_items > 448
    _run_compare(w, seqs=[0, 13, 39], heads=[0, 7, 15])


FP32_MODE = [
    small_variant(V2, name="v2_fp32mode_split3", batch=3, kv_len=0, lengths=(700, 64, 1),
                  num_splits=3),
    small_variant(V2, name="fp8_fp32mode_t4", batch=2, q_tokens=4, kv_len=0, lengths=(300, 9),
                  kv_dtype="fp8"),
]


@pytest.mark.parametrize("w", FP32_MODE, ids=[w.name for w in FP32_MODE])
def test_decode_parity_fp32_mode(w):
    _run_compare(w, precision="fp32")


# ------------------------------------------------- full-size workloads
# Full-size workloads: 8 sequences (all 4 of the long-context one) and 16
# heads or more, every 8th head plus head 127 (each of the four 32-row waves of
# a 128-row block), and the 8 rows of largest |o|.
_H16 = list(range(0, 128, 8)) + [127]
FULL = [
    (WORKLOADS["v2_b32_l4k_bf16"], [0, 4, 9, 13, 17, 22, 26, 31], _H16),
    (WORKLOADS["v2_b64_l8k_bf16"], [0, 5, 14, 23, 32, 41, 50, 63], _H16),
    (WORKLOADS["v2_fp8_t4_b64_l8k"], [0, 9, 18, 27, 36, 45, 54, 63], _H16),
    (WORKLOADS["v2_fp6_t4_b64_l8k"], [0, 9, 18, 27, 36, 45, 54, 63], _H16),
    (WORKLOADS["v2_long_b4_l128k_bf16"], [0, 1, 2, 3], [0, 8, 16, 24, 40, 56, 64, 72, 77, 88,
                                                        96, 104, 112, 120, 127, 33]),
    (WORKLOADS["v2lite_b64_l8k_bf16"], [0, 9, 18, 27, 31, 45, 54, 63], list(range(16))),
]


@pytest.mark.parametrize("w,seqs,heads", FULL, ids=[f[0].name for f in FULL])
def test_decode_parity_full_size(w, seqs, heads):
    _run_compare(w, seqs=seqs, heads=heads, top_abs=8)


def test_bf16_mode_on_outlier_workloads():
    """The bf16-operand path alone (precision BF16: no recomputation) on the
    outlier workloads: within the rel-L2 gate; its max-abs error is what the
    split operands remove (both gates hold in the default mode above)."""
    w = SMALL[[x.name for x in SMALL].index("v2_outliers_split7")]
    _run_compare(w, precision="bf16", max_abs=False)
    w = WORKLOADS["v2_long_b4_l128k_bf16"]
    _run_compare(w, seqs=[0, 3], heads=[0, 77, 127], precision="bf16", max_abs=False)


# The split-operand kernel on every item (precision BF16X2), both gates.
X2 = [
    small_variant(V2, name="x2_ragged_split5", batch=4, kv_len=0, lengths=(1, 33, 700, 64),
                  num_splits=5),
    small_variant(V2, name="x2_paged", batch=5, kv_len=0, lengths=(40, 900, 64, 65, 333),
                  layout="paged"),
    small_variant(V2, name="x2_t4_causal", batch=3, q_tokens=4, kv_len=0, lengths=(300, 4, 130),
                  num_splits=2),
    small_variant(V2, name="x2_outliers_split3", batch=2, kv_len=0, lengths=(3000, 2900),
                  num_splits=3, outlier_frac=0.01, outlier_scale=8.0),
    small_variant(V2, name="x2_rope_yarn", batch=2, kv_len=0, lengths=(4600, 900), rope=True,
                  yarn_factor=40.0),
]


@pytest.mark.parametrize("w", X2, ids=[w.name for w in X2])
def test_decode_parity_split_operands(w):
    heads = [0, 31, 64, 127] if w.rope else None
    _run_compare(w, heads=heads, precision="bf16x2")


def _latent_lse(w, gen, precision, num_splits=None):
    buf = _buffers(w, gen, precision=precision, num_splits=num_splits)
    buf.absorb()
    buf.attend()
    torch.cuda.synchronize()
    return to_np(buf.latent), to_np(buf.lse)


def test_escalation_decisions():
    """AUTO escalates exactly the items that need it.  On N(0,1) data (largest
    scores ~4-5) no item is recomputed: the result is bit for bit that of the
    bf16-operand path.  With 1% of the cache rows scaled by 8 every item holds
    scores far past the threshold: the result is bit for bit that of the
    split-operand path (same kernel, same fp32 partials, same combine)."""
    w = small_variant(V2, name="esc_plain", batch=3, kv_len=0, lengths=(3000, 700, 1500),
                      num_splits=3)
    gen = generate(w)
    a_lat, a_lse = _latent_lse(w, gen, "auto")
    b_lat, b_lse = _latent_lse(w, gen, "bf16")
    assert np.array_equal(a_lat, b_lat) and np.array_equal(a_lse, b_lse)
    w = small_variant(V2, name="esc_outliers", batch=2, kv_len=0, lengths=(3000, 2900),
                      num_splits=3, outlier_frac=0.01, outlier_scale=8.0)
    gen = generate(w)
    a_lat, a_lse = _latent_lse(w, gen, "auto")
    x_lat, x_lse = _latent_lse(w, gen, "bf16x2")
    assert np.array_equal(a_lat, x_lat) and np.array_equal(a_lse, x_lse)
    b_lat, _ = _latent_lse(w, gen, "bf16")
    assert not np.array_equal(a_lat, b_lat)


def test_decode_parity_full_size_paged():
    w = WORKLOADS["v2_paged_b128_bf16"]
    gen = generate(w)
    L = gen["seq_lens"]
    seqs = sorted({int(np.argmin(L)), int(np.argmax(L)), 5, 20, 47, 66, 93, 120})
    _run_compare(w, gen=gen, seqs=seqs, heads=_H16, top_abs=8)


# ------------------------------------------------------ properties
@pytest.mark.parametrize("precision", ["bf16", "bf16x2"])
def test_split_invariance_and_determinism(precision):
    w = small_variant(V2, name="split_inv", batch=2, kv_len=0, lengths=(2000, 1500))
    gen = generate(w)
    ref = omla.decode_workload(gen, w)
    outs = {}
    for ns in (1, 2, 7, 0):
        buf = _buffers(w, gen, num_splits=ns, precision=precision)
        buf.step()
        torch.cuda.synchronize()
        outs[ns] = (to_np(buf.latent), to_np(buf.o))
        check(f"latent splits={ns}", outs[ns][0], ref["latent"], REL_L2_BF16, MAX_ABS_BF16)
        buf.step()                                    # same plan again: bitwise equal
        torch.cuda.synchronize()
        assert np.array_equal(to_np(buf.latent), outs[ns][0])
        assert np.array_equal(to_np(buf.o), outs[ns][1])
    # bf16 operands: a split run stores each chunk's partial latent in bf16
    # before the LSE combine, one extra rounding of at most 2^-8 relative per
    # element on top of the unsplit result, whose own operands are bf16: the
    # two may differ by up to about one bf16 unit roundoff (2^-8) in rel-L2.
    # Split operands: fp32 partials and ~2^-17 operand errors; the split and
    # unsplit results differ only by fp32 rounding in the combine and in the
    # accumulation order (bound 1e-5).
    bound = 2.0 ** -8 if precision == "bf16" else 1e-5
    for ns in (2, 7, 0):
        r = rel_l2(outs[ns][0], outs[1][0])
        say(f"  splits={ns} vs unsplit: rel-L2 {r:.2e}")
        assert r <= bound


def test_paged_equals_contiguous_bitwise():
    """Token order is logical order whatever the physical page order, so the
    same plan gives bitwise-identical results (token permutation invariance
    of the page table)."""
    base = small_variant(V2, name="perm", batch=3, kv_len=0, lengths=(700, 64, 200))
    gen = generate(base)
    paged = dataclasses.replace(base, layout="paged")
    genp = generate(paged)
    for k in ("c_kv", "k_r", "q_nope", "q_rope", "w_uk", "w_uv"):
        assert np.array_equal(gen[k], genp[k])
    a = _buffers(base, gen)
    b = _buffers(paged, genp)
    a.step()
    b.step()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(a.latent), to_np(b.latent))
    assert np.array_equal(to_np(a.o), to_np(b.o))


def test_reference_restart_on_large_score_jump():
    """A late token whose score exceeds the first tile's max by far more than
    2^64 (log2 units) forces the matrix-core kernel to restart its work item
    with a higher reference; the result must still match the oracle.  The
    rows scaled by 64 scale the bf16 operand rounding by 64 as well, so the
    bf16-operand path is held to the rel-L2 gate, the split-operand and fp32
    paths to both gates.
    For several heads the jump exceeds 128 (log2 units): without the restart
    their weights would overflow fp32, so a missed restart shows up as a
    non-finite output."""
    w = small_variant(V2, name="restart", batch=2, kv_len=0, lengths=(1000, 900))
    gen = generate(w)
    c = formats.bf16_to_f64(gen["c_kv"])
    c[700] *= 64.0                  # sequence 0, late tile
    c[1000 + 500] *= 64.0           # sequence 1
    from mla_inputs import bf16_bits_from_f32
    gen["c_kv"] = bf16_bits_from_f32(c.astype(np.float32))
    _run_compare(w, gen=gen, precision="bf16", max_abs=False)   # restart of the bf16 kernel
    _run_compare(w, gen=gen)        # AUTO: recomputed (and restarted) with split operands
    _run_compare(w, gen=gen, precision="bf16x2")
    _run_compare(w, gen=gen, precision="fp32")


@pytest.mark.parametrize("kv", ["fp8", "fp6"])
def test_reference_restart_quantised_caches(kv):
    """The restart of the quantised-cache kernels: rows scaled by 64 before
    the cache is written (their scale absorbs the factor), late in each
    sequence, with T = 4 causal rows; the fp8 kernel answers a restart with
    a pass that finds every row's largest score and a second pass from that
    reference.  The quantised caches are held to their rel-L2 gate."""
    w = small_variant(V2, name=f"restart_{kv}", batch=2, q_tokens=4, kv_len=0,
                      lengths=(1000, 900), kv_dtype=kv)
    gen = generate(w)
    c = formats.bf16_to_f64(gen["c_kv"])
    c[700] *= 64.0
    c[1000 + 500] *= 64.0
    from mla_inputs import bf16_bits_from_f32
    gen["c_kv"] = bf16_bits_from_f32(c.astype(np.float32))
    _run_compare(w, gen=gen, max_abs=False)


# --------------------------------------------------- append, bit exact
@pytest.mark.parametrize("layout", ["contiguous", "paged"])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp6", "f32"])
def test_cache_append_bit_exact(layout, kv):
    w = small_variant(V2, name=f"append_{kv}_{layout}", batch=3, kv_len=0,
                      lengths=(65, 200, 3), layout=layout, kv_dtype=kv,
                      q_dtype="f32" if kv == "f32" else "bf16")
    say(f"case append kv={kv} layout={layout}")
    gen = generate(w)
    buf = _buffers(w, gen)
    torch.cuda.synchronize()
    rows = omla.cache_row_index(gen["row_seq"], gen["row_pos"], gen.get("page_table"),
                                w.page_size, buf.max_len)
    cache = buf.cache.cpu()
    if kv == "fp8":
        d = omla.logical_inputs(gen, w)
        got = cache.numpy()[rows]
        assert np.array_equal(got, d["fp8_codes"])
        assert np.array_equal(buf.kv_scale.cpu().numpy()[rows], d["fp8_scales"])
    elif kv == "fp6":
        d = omla.logical_inputs(gen, w)
        got = cache.numpy()[rows]
        assert np.array_equal(got, formats.pack_rows_mxfp6(d["fp6_codes"], d["fp6_exps"]))
    elif kv == "bf16":
        got = cache.view(torch.int16).numpy().view(np.uint16)[rows]
        assert np.array_equal(got, np.concatenate([gen["c_kv"], gen["k_r"]], 1))
    else:
        got = cache.numpy()[rows]
        assert np.array_equal(got, np.concatenate([gen["c_kv"], gen["k_r"]], 1))
    # every slot not written must still hold the NaN poison
    written = np.zeros(buf.cache_rows, dtype=bool)
    written[rows] = True
    rest = cache.numpy()[~written] if kv != "bf16" else cache.float().numpy()[~written]
    if kv == "fp8":
        assert np.all(rest == 0x7F)
    elif kv == "fp6":
        assert np.all(rest == 0xFF)
    else:
        assert np.all(np.isnan(rest))


@pytest.mark.parametrize("w", [WORKLOADS["tiny_fp32"],
                               small_variant(WORKLOADS["tiny_fp32"], name="tiny_fp32_yarn",
                                             yarn_factor=8.0, yarn_orig_len=16,
                                             yarn_beta=8.0)],
                         ids=["plain", "yarn"])
def test_cache_append_rope_matches_oracle(w):
    gen = generate(w)
    buf = _buffers(w, gen)
    torch.cuda.synchronize()
    d = omla.logical_inputs(gen, w)
    got = buf.cache.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got[:, :w.d_latent], d["c_rows"], rtol=0, atol=0)
    np.testing.assert_allclose(got[:, w.d_latent:], d["kr_rows"], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("n_heads", [128, 16], ids=["rows128", "rows16"])
def test_fp8_every_code_decodes_exactly(n_heads):
    """L = 1: the softmax weight is exactly 1, so the latent output is the
    stored row itself; rows built from all 254 finite E4M3 codes with scale 1
    must come back as their exact values (both attention kernels)."""
    from head_latent_attention_11_amd.runner import DecodeBuffers
    w = small_variant(V2, name="codes", batch=2, kv_len=0, lengths=(1, 1), kv_dtype="fp8",
                      n_heads=n_heads)
    gen = generate(w)
    buf = DecodeBuffers(w, gen)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    row = np.zeros((2, 576), dtype=np.uint8)
    row[0, :254] = codes
    row[1, :254] = codes[::-1]
    row[:, 254:508] = codes
    row[:, 508:512] = codes[:4]
    buf.cache[:2] = torch.from_numpy(row).cuda()
    buf.kv_scale[:2] = 1.0
    buf.absorb()                      # no append: the cache holds the rows written above
    buf.attend()
    buf.up_proj()
    torch.cuda.synchronize()
    lat = to_np(buf.latent)                       # [2, n_h, 512]
    exp = formats.e4m3_to_f64(row[:, :512])
    for b in range(2):
        assert np.array_equal(lat[b], np.broadcast_to(exp[b], lat[b].shape)), b


def test_fp6_every_code_decodes_exactly():
    """L = 1: the latent output is the stored row itself.  Rows built from
    all 64 E2M3 codes under block exponents from -20 to +20 (18 blocks a
    row) must come back as their exact values.  The query is zero, so every
    score is 0 and the weight exactly 1 (with rows this large a nonzero
    query gives scores near 1e8, where the weight 2^(s - max) is 1 only to
    within the rounding of s)."""
    from head_latent_attention_11_amd.runner import DecodeBuffers
    w = small_variant(V2, name="codes6", batch=2, kv_len=0, lengths=(1, 1), kv_dtype="fp6")
    gen = generate(w)
    buf = DecodeBuffers(w, gen)
    codes = np.zeros((2, 576), dtype=np.uint8)
    codes[0] = np.arange(576) % 64
    codes[1] = (63 - np.arange(576)) % 64
    exps = np.zeros((2, 18), dtype=np.int32)
    exps[0] = np.arange(18) - 9
    exps[1] = np.linspace(-20, 20, 18).astype(np.int32)
    row = formats.pack_rows_mxfp6(codes, exps)
    rows = omla.cache_row_index(np.array([0, 1]), np.array([0, 0]), None, 64, buf.max_len)
    for r in range(2):
        buf.cache[int(rows[r])] = torch.from_numpy(row[r]).cuda()
    buf.q_nope.zero_()
    buf.q_rope.zero_()
    buf.absorb()                      # no append: the cache holds the rows written above
    buf.attend()
    torch.cuda.synchronize()
    lat = to_np(buf.latent)
    exp = formats.dequantize_rows_mxfp6(codes, exps)[:, :512]
    for b in range(2):
        assert np.array_equal(lat[b], np.broadcast_to(exp[b], lat[b].shape)), b


# ------------------------------------------- absorb and up-projection
@pytest.mark.parametrize("w", [V2, WORKLOADS["tiny_fp32"],
                               small_variant(V2, name="n16", n_heads=16),
                               small_variant(V2, name="n16_t3", n_heads=16, q_tokens=3,
                                             rope=True, yarn_factor=40.0)],
                         ids=["v2_mfma", "tiny_fp32_rope", "n16_mfma", "n16_111_tokens_yarn"])
def test_absorb_q_parity(w):
    w = small_variant(w, batch=min(w.batch, 37), kv_len=0, lengths=(64,) * min(w.batch, 37))
    gen = generate(w)
    buf = _buffers(w, gen)
    buf.absorb()
    torch.cuda.synchronize()
    d = omla.logical_inputs(gen, w)
    ref = omla.absorbed_query(d["q_nope"], d["q_rope"], d["w_uk"])
    got = to_np(buf.q_abs)
    if buf.dims.qabs_pairs():
        # (hi, lo) pairs: hi is the bf16 rounding of the fp32 result and
        # hi + lo carries it to ~2^-17 relative (fp32 accumulation beyond)
        hi, lo = got[:, :, 0, :], got[:, :, 1, :]
        check("q_abs hi", hi, ref, 4e-3)
        assert np.all(np.abs(lo) <= np.abs(hi) * 2.0 ** -8 + 1e-30)
        check("q_abs hi + lo", hi + lo, ref, 2e-5)
        # elementwise: the lo rounding (2^-17 |q|) plus the fp32 accumulation
        # of 128 products (at most 128 * 2^-24 of the sum of their
        # magnitudes); the rotated RoPE part is a single fp32 rounding away
        mag = np.abs(ref).copy()
        for i in range(w.n_heads):
            mag[:, i, :w.d_latent] = np.abs(d["q_nope"][:, i, :]) @ np.abs(d["w_uk"][i])
        bound = 2.0 ** -17 * np.abs(ref) + 128 * 2.0 ** -24 * mag + 2.0 ** -24 * np.abs(ref)
        assert np.all(np.abs(hi + lo - ref) <= 2 * bound + 1e-30)
        return
    # q_abs is stored in the query format: bf16 rounding (2^-9 relative)
    tol = 1e-6 if w.q_dtype == "f32" else 4e-3
    check("q_abs", got, ref, tol)
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 1e-3)) < (1e-5 if w.q_dtype == "f32" else 8e-3)


@pytest.mark.parametrize("w", [V2, WORKLOADS["tiny_fp32"],
                               small_variant(V2, name="n16", n_heads=16)],
                         ids=["v2_mfma", "tiny_fp32", "n16_mfma"])
def test_up_proj_parity(w):
    """Latent inputs are drawn here (seeded), never taken from the HIP path."""
    n_tok = 45
    rng = np.random.default_rng(77)
    latent = (rng.standard_normal((n_tok, w.n_heads, w.d_latent)) * 0.05).astype(np.float32)
    gen = generate(small_variant(w, batch=1, kv_len=64, lengths=()))
    from head_latent_attention_11_amd import binding as B
    from head_latent_attention_11_amd.runner import to_device
    dims = B.MLADims.from_workload(w)
    kind = "f32" if w.q_dtype == "f32" else "bf16"
    w_uv = to_device(gen["w_uv"], kind, "cuda")
    lat_d = torch.from_numpy(latent).cuda()
    out = torch.full((n_tok, w.n_heads, w.d_head), float("nan"), dtype=w_uv.dtype, device="cuda")
    out32 = torch.full((n_tok, w.n_heads, w.d_head), float("nan"), dtype=torch.float32,
                       device="cuda")
    B.up_proj_v(dims, lat_d, w_uv, out, n_tok)
    B.up_proj_v(dims, lat_d, w_uv, out32, n_tok)
    torch.cuda.synchronize()
    w_uv64 = formats.bf16_to_f64(gen["w_uv"]) if kind == "bf16" else gen["w_uv"].astype(np.float64)
    ref = omla.up_project(latent.astype(np.float64), w_uv64)
    got = to_np(out)
    check("o", got, ref, 1e-6 if kind == "f32" else 4e-3)
    check("o (fp32 out)", to_np(out32), ref, 1e-5)


# ------------------------------------------ the benchmark's launch configuration
@pytest.mark.parametrize("w", [V2,
                               small_variant(WORKLOADS["v2_fp8_t4_b64_l8k"], name="fp8_t4_graph",
                                             batch=5, kv_len=0, lengths=(700, 64, 4, 333, 1200)),
                               small_variant(WORKLOADS["v2_paged_b128_bf16"], name="paged_graph",
                                             batch=6, kv_len=0,
                                             lengths=(513, 64, 2000, 1, 65, 900)),
                               small_variant(WORKLOADS["v2lite_b64_l8k_bf16"], name="lite_graph",
                                             batch=6, kv_len=0,
                                             lengths=(513, 64, 2000, 1, 65, 900),
                                             layout="paged"),
                               small_variant(WORKLOADS["v2lite_b64_l8k_bf16"], name="lite_fp8_graph",
                                             batch=5, kv_len=0, q_tokens=2,
                                             lengths=(700, 64, 4, 333, 1200), kv_dtype="fp8")],
                         ids=["v2_b32_l4k_bf16", "fp8_t4_ragged", "paged_ragged", "lite_paged_ragged",
                              "lite_fp8_t2_ragged"])
def test_graph_replays_match_eager(w):
    """Steps captured as one HIP graph over two cache replicas (as the
    benchmark runs them) give, on every replay, the eager step's outputs bit
    for bit; the outputs are poisoned with NaN by eager work between replays.
    The eager step itself is checked against the oracle on sampled rows."""
    say(f"case graph {w.name}: B={w.batch} T={w.q_tokens} kv={w.kv_dtype} layout={w.layout}")
    gen = generate(w)
    buf = _buffers(w, gen, cache_replicas=2)
    buf.step(replica=0)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (buf.o, buf.latent, buf.lse)]
    seqs = sorted({0, w.batch - 1})
    ref = omla.decode_workload(gen, w, seqs=seqs, heads=[0, w.n_heads - 1])
    mask = sample_mask((w.batch * w.q_tokens, w.n_heads), seqs, [0, w.n_heads - 1], w.q_tokens)
    rel, mabs = _gates(w)
    check("o (eager)", to_np(eager[0])[mask], ref["o"][mask], rel, mabs)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        buf.step(replica=1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for r in (1, 0, 1, 0):                 # the last step reads replica 0
            buf.step(replica=r)
    for rep in range(3):
        for t in (buf.o, buf.latent, buf.lse):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "latent", "lse"), (buf.o, buf.latent, buf.lse), eager):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
    say(f"  3 replays bit-identical to the eager step")



# ------------------------------------------- output projection u = W^O [o_1; ...]
OUT_PROJ = [
    (V2, 32, "f32"),            # the benchmark's 32 tokens, one token tile
    (V2, 45, "bf16"),           # a ragged second token tile, bf16 output
    (V2, 200, "f32"),           # two token groups (128 + 72)
    (small_variant(V2, name="v2_d256", d_model=256), 7, "f32"),
    (small_variant(V2, name="v2_d640", d_model=640), 300, "bf16"),   # groups of 256 + 44 tokens
    (WORKLOADS["tiny_fp32"], 5, "f32"),                           # general path (fp32)
    (small_variant(V2, name="v2_d200", d_model=200), 9, "bf16"),  # general path (d % 128 != 0)
]


@pytest.mark.parametrize("w,n_tok,u_kind", OUT_PROJ,
                         ids=[f"{c[0].name}-{c[1]}-{c[2]}" for c in OUT_PROJ])
def test_out_proj_parity(w, n_tok, u_kind):
    """u = W^O [o_1; ...; o_{n_h}] through the C ABI against the oracle, on all
    outputs; o is drawn here (seeded) in the query format, W^O by the input
    generator; u in fp32 or bf16."""
    from head_latent_attention_11_amd import binding as B
    from head_latent_attention_11_amd.runner import to_device
    from mla_inputs import output_weights
    say(f"case out_proj {w.name}: n_tok={n_tok} d_model={w.d_model} K={w.n_heads * w.d_head} "
        f"u={u_kind}")
    kind = "f32" if w.q_dtype == "f32" else "bf16"
    rng = np.random.default_rng(91)
    o32 = rng.standard_normal((n_tok, w.n_heads, w.d_head)).astype(np.float32)
    from mla_inputs import bf16_bits_from_f32
    o_st = o32 if kind == "f32" else bf16_bits_from_f32(o32)
    w_o = output_weights(w)
    dims = B.MLADims.from_workload(w)
    o_d = to_device(o_st, kind, "cuda")
    w_d = to_device(w_o, kind, "cuda")
    udt = torch.float32 if u_kind == "f32" else torch.bfloat16
    u = torch.full((n_tok, w.d_model), float("nan"), dtype=udt, device="cuda")
    o_code = B.F32 if kind == "f32" else B.BF16
    wsb = B.out_proj_workspace_size(dims, w.d_model, n_tok, o_code)
    ws = (torch.full(((wsb + 15) // 16 * 4,), float("nan"), dtype=torch.float32, device="cuda")
          if wsb else None)
    B.out_proj(dims, o_d, w_d, w.d_model, u, n_tok, ws, wsb)
    torch.cuda.synchronize()
    got = to_np(u)
    assert np.all(np.isfinite(got))
    o64 = o_st.astype(np.float64) if kind == "f32" else formats.bf16_to_f64(o_st)
    w64 = w_o.astype(np.float64) if kind == "f32" else formats.bf16_to_f64(w_o)
    ref = omla.output_project(o64, w64)
    # exact bf16 products, fp32 sums over K = n_h d_h; bf16 output adds 2^-9
    check("u", got, ref, 1e-5 if u_kind == "f32" else 4e-3)



OUT_PROJ_PACKED = [
    (V2, 32, "f32"),            # one token tile, 5-wave workgroups
    (V2, 45, "bf16"),           # a ragged second token tile (groups of 4 tiles)
    (V2, 256, "f32"),           # groups of 8 token tiles
    (small_variant(V2, name="v2_d256", d_model=256), 7, "f32"),      # 128-row feature blocks
    (small_variant(V2, name="v2_d352", d_model=352), 300, "bf16"),   # partial last block
]


def _panel_layout(w_rm):
    """The documented panel layout of mla_out_proj_packed, from the row-major
    matrix: element (f, k) at ((f/32)(K/64) + k/64) 2048 + (f%32) 64 + k%64."""
    d, K = w_rm.shape
    return w_rm.reshape(d // 32, 32, K // 64, 64).transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("w,n_tok,u_kind", OUT_PROJ_PACKED,
                         ids=[f"{c[0].name}-{c[1]}-{c[2]}" for c in OUT_PROJ_PACKED])
def test_out_proj_packed_parity(w, n_tok, u_kind):
    """mla_out_proj_pack writes the documented panel layout (bit-exact), and
    mla_out_proj_packed gives the same u, bit for bit, as mla_out_proj on the
    row-major W^O, and matches the oracle."""
    from head_latent_attention_11_amd import binding as B
    from head_latent_attention_11_amd.runner import to_device
    from mla_inputs import bf16_bits_from_f32, output_weights
    say(f"case out_proj_packed {w.name}: n_tok={n_tok} d_model={w.d_model} u={u_kind}")
    rng = np.random.default_rng(93)
    o_st = bf16_bits_from_f32(rng.standard_normal((n_tok, w.n_heads, w.d_head)).astype(np.float32))
    w_o = output_weights(w)
    dims = B.MLADims.from_workload(w)
    o_d = to_device(o_st, "bf16", "cuda")
    w_d = to_device(w_o, "bf16", "cuda")
    w_p = torch.full_like(w_d, float("nan"))
    B.out_proj_pack(dims, w_d, w.d_model, w_p)
    torch.cuda.synchronize()
    got_p = w_p.view(torch.int16).cpu().numpy().reshape(-1)
    assert np.array_equal(got_p, _panel_layout(w_o.view(np.int16))), "panel layout differs"
    udt = torch.float32 if u_kind == "f32" else torch.bfloat16
    wsb = B.out_proj_workspace_size(dims, w.d_model, n_tok, B.BF16)
    ws = torch.full(((wsb + 15) // 16 * 4,), float("nan"), dtype=torch.float32, device="cuda")
    u_p = torch.full((n_tok, w.d_model), float("nan"), dtype=udt, device="cuda")
    u_r = torch.full((n_tok, w.d_model), float("nan"), dtype=udt, device="cuda")
    B.out_proj_packed(dims, o_d, w_p, w.d_model, u_p, n_tok, ws, wsb)
    torch.cuda.synchronize()
    B.out_proj(dims, o_d, w_d, w.d_model, u_r, n_tok, ws, wsb)
    torch.cuda.synchronize()
    assert torch.equal(u_p, u_r), "packed and row-major projections differ"
    ref = omla.output_project(formats.bf16_to_f64(o_st), formats.bf16_to_f64(w_o))
    check("u", to_np(u_p), ref, 1e-5 if u_kind == "f32" else 4e-3)


# ------------------------------ cache producer: [RMSNorm(W^DKV h) ; RoPE(W^KR h)]
PRODUCE = [
    (V2, "contiguous", True),
    (small_variant(V2, name="v2_fp8", kv_dtype="fp8"), "paged", True),
    (V2, "paged", False),                                          # no RMS norm
    (WORKLOADS["tiny_fp32"], "contiguous", True),                  # fp32: general projection
    (small_variant(V2, name="v2_yarn", yarn_factor=40.0, yarn_orig_len=64), "paged", True),
]


@pytest.mark.parametrize("w,layout,norm", PRODUCE,
                         ids=[f"{c[0].name}-{c[1]}-{'norm' if c[2] else 'nonorm'}" for c in PRODUCE])
def test_kv_produce_parity(w, layout, norm):
    """mla_kv_produce through the C ABI: the rows it writes into a NaN-poisoned
    cache against the oracle's rows of the same hidden states (stored in the
    cache's format: bf16 rounding, fp8 codes times the row scale, fp32);
    every other slot stays untouched."""
    from head_latent_attention_11_amd import binding as B
    from head_latent_attention_11_amd.runner import to_device
    from mla_inputs import producer_inputs
    say(f"case kv_produce {w.name}: layout={layout} kv={w.kv_dtype} norm={norm}")
    n_seq, max_len = 5, 192
    rng = np.random.default_rng(61)
    n_rows = 45
    seq = rng.integers(0, n_seq, size=n_rows).astype(np.int32)
    pos = np.empty(n_rows, dtype=np.int32)
    for s_ in range(n_seq):                                   # distinct positions per sequence
        idx = np.nonzero(seq == s_)[0]
        pos[idx] = rng.choice(max_len, size=len(idx), replace=False)
    inp = producer_inputs(w, n_rows)
    D = w.d_latent + w.d_rope
    kind = "f32" if w.q_dtype == "f32" else "bf16"
    dims = B.MLADims.from_workload(w)
    if layout == "paged":
        pages_per_seq = max_len // 64
        table = rng.permutation(n_seq * pages_per_seq).astype(np.int32).reshape(n_seq, -1)
        pt, max_pages, ml = torch.from_numpy(table).cuda(), pages_per_seq, 0
        slot = table[seq, pos // 64].astype(np.int64) * 64 + pos % 64
    else:
        pt, max_pages, ml = None, 0, max_len
        slot = seq.astype(np.int64) * max_len + pos
    n_slots = n_seq * max_len
    if w.kv_dtype == "fp8":
        cache = torch.full((n_slots, D), 0x7F, dtype=torch.uint8, device="cuda")
        scale = torch.full((n_slots,), float("nan"), dtype=torch.float32, device="cuda")
    else:
        cache = torch.full((n_slots, D), float("nan"),
                           dtype=torch.float32 if w.kv_dtype == "f32" else torch.bfloat16,
                           device="cuda")
        scale = None
    gain = torch.from_numpy(inp["gain"]).cuda() if norm else None
    eps = 1e-6
    wsb = B.kv_produce_workspace_size(dims, w.d_model, n_rows)
    ws = torch.full(((wsb + 15) // 16 * 4,), float("nan"), dtype=torch.float32, device="cuda")
    B.kv_produce(dims, to_device(inp["h"], kind, "cuda"), w.d_model,
                 to_device(inp["w_dkv_kr"], kind, "cuda"), gain, eps,
                 torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), pt, n_seq, max_pages,
                 ml, n_slots, True, cache, scale, n_rows, ws, wsb)
    torch.cuda.synchronize()
    h64 = inp["h"].astype(np.float64) if kind == "f32" else formats.bf16_to_f64(inp["h"])
    w64 = (inp["w_dkv_kr"].astype(np.float64) if kind == "f32"
           else formats.bf16_to_f64(inp["w_dkv_kr"]))
    ref = omla.produce_rows(h64, w64[:w.d_latent], w64[w.d_latent:],
                            inp["gain"].astype(np.float64) if norm else None, eps, pos=pos,
                            theta=yarn_theta(w.d_rope, w.rope_base, w.yarn_factor,
                                             w.yarn_alpha, w.yarn_beta, w.yarn_orig_len))
    if w.kv_dtype == "fp8":
        codes = cache.cpu().numpy()
        sc = scale.cpu().numpy()
        got = formats.e4m3_to_f64(codes[slot]) * sc[slot][:, None]
        written = np.zeros(n_slots, dtype=bool)
        written[slot] = True
        assert np.all(np.isnan(sc[~written])), "a slot outside the new rows was written"
        check("rows (fp8)", got, ref, REL_L2_FP8)
        # against the oracle's rows stored the same way (per-row scale, E4M3
        # codes): the fp32 projection moves only codes at a rounding boundary
        qc, qs = formats.quantize_rows_e4m3(ref.astype(np.float32))
        check("rows (fp8, both quantised)", got, formats.dequantize_rows_e4m3(qc, qs), 5e-3)
    else:
        c = to_np(cache)
        got = c[slot]
        written = np.zeros(n_slots, dtype=bool)
        written[slot] = True
        assert np.all(np.isnan(c[~written])), "a slot outside the new rows was written"
        check("rows", got, ref, 1e-5 if w.kv_dtype == "f32" else 4e-3)


# ------------------------------------------------------ debug aids
def _page_check_expected(pt, lens, n_pages):
    """Host count of the page-table check: out-of-range ids among each row's
    used entries (all entries when the length is out of range)."""
    batch, max_pages = pt.shape
    count, first, badlen = 0, -1, 0
    for b in range(batch):
        L = int(lens[b])
        ok = 0 <= L <= max_pages * 64
        badlen += 0 if ok else 1
        used = (L + 63) // 64 if ok else max_pages
        for p in range(used):
            v = int(pt[b, p])
            if v < 0 or v >= n_pages:
                count += 1
                if first < 0:
                    first = b * max_pages + p
    return [count, first, int(pt.reshape(-1)[first]) if count else 0, badlen]


@pytest.mark.parametrize("batch,max_pages,n_pages", [(37, 50, 900), (1000, 600, 100000)])
def test_page_table_check(batch, max_pages, n_pages):
    """mla_check_page_table on a valid table, then with out-of-range ids
    planted in used entries (counted), in unused entries past a sequence's
    length (not counted) and with out-of-range lengths."""
    from head_latent_attention_11_amd import binding as B
    say(f"case page check: batch={batch} max_pages={max_pages} n_pages={n_pages}")
    dims = B.MLADims.make(128, 128, 512, 64)
    rng = np.random.default_rng(batch)
    lens = rng.integers(1, max_pages * 64 + 1, size=batch).astype(np.int32)
    pt = rng.integers(0, n_pages, size=(batch, max_pages)).astype(np.int32)
    result = torch.full((4,), 12345, dtype=torch.int32, device="cuda")

    def run(pt_h, lens_h):
        B.check_page_table(dims, torch.from_numpy(pt_h).cuda(), max_pages,
                           torch.from_numpy(lens_h).cuda(), batch, n_pages, result)
        torch.cuda.synchronize()
        return result.cpu().tolist()

    assert run(pt, lens) == [0, -1, 0, 0]
    bad = pt.copy()
    lens2 = lens.copy()
    used = (lens2 + 63) // 64
    for k, b in enumerate(rng.choice(batch, size=min(batch, 12), replace=False)):
        p = int(rng.integers(0, used[b]))
        bad[b, p] = [-1, n_pages, n_pages + 7, -(1 << 30)][k % 4]
        if used[b] < max_pages:                       # past the length: not read, not counted
            bad[b, int(used[b])] = -5
    lens2[rng.integers(0, batch)] = -3
    lens2[rng.integers(0, batch)] = max_pages * 64 + 1
    want = _page_check_expected(bad, lens2, n_pages)
    got = run(bad, lens2)
    say(f"  planted: got {got}, host count {want}")
    assert got == want and got[0] > 0


GUARD = 4096
GUARD_BYTE = 0xA5


def _guarded_like(t):
    """A tensor of t's shape, dtype and contents inside a larger allocation
    whose GUARD bytes before and after hold a fixed byte."""
    nbytes = t.numel() * t.element_size()
    raw = torch.full((nbytes + 2 * GUARD,), GUARD_BYTE, dtype=torch.uint8, device=t.device)
    view = raw[GUARD:GUARD + nbytes].view(t.dtype).view(t.shape)
    view.copy_(t)
    return raw, view


@pytest.mark.parametrize("w", [
    small_variant(V2, name="canary_split5", batch=4, kv_len=0, lengths=(1, 33, 700, 64),
                  num_splits=5),
    small_variant(V2, name="canary_split40_paged", batch=3, kv_len=0, lengths=(2600, 64, 1300),
                  num_splits=40, layout="paged"),
    small_variant(V2, name="canary_fp8_t4", batch=4, q_tokens=4, kv_len=0,
                  lengths=(300, 77, 4, 130), kv_dtype="fp8", num_splits=3),
    small_variant(V2, name="canary_lite_n16", batch=4, n_heads=16, kv_len=0,
                  lengths=(1, 33, 700, 64), num_splits=4),
], ids=lambda w: w.name)
def test_output_guard_canaries(w):
    """Every buffer a decode step writes (absorbed query, cache with its
    scales, split workspace, latent, LSE, output) sits between guard bytes;
    after the step the guards are unchanged and the output still passes the
    oracle comparison."""
    say(f"case canaries {w.name}: B={w.batch} T={w.q_tokens} kv={w.kv_dtype} layout={w.layout}")
    gen = generate(w)
    buf = _buffers(w, gen)
    raws = {}
    for name in ("q_abs", "latent", "lse", "o"):
        raws[name], view = _guarded_like(getattr(buf, name))
        setattr(buf, name, view)
    if buf.workspace is not None:
        raws["workspace"], buf.workspace = _guarded_like(buf.workspace)
    raws["cache"], buf.caches[0] = _guarded_like(buf.caches[0])
    if buf.scales[0] is not None:
        raws["scales"], buf.scales[0] = _guarded_like(buf.scales[0])
    buf.step()
    torch.cuda.synchronize()
    for name, raw in raws.items():
        head = raw[:GUARD].cpu().numpy()
        tail = raw[-GUARD:].cpu().numpy()
        assert np.all(head == GUARD_BYTE) and np.all(tail == GUARD_BYTE), f"{name}: guard overwritten"
    ref = omla.decode_workload(gen, w)
    rel, mabs = _gates(w)
    check("o", to_np(buf.o), ref["o"], rel, mabs)


@pytest.mark.parametrize("w", [
    small_variant(V2, name="aa_bf16_pairs", batch=4, kv_len=0, lengths=(1, 33, 700, 64)),
    small_variant(V2, name="aa_fp8_t4", batch=4, q_tokens=4, kv_len=0, lengths=(300, 77, 4, 130),
                  kv_dtype="fp8"),
    small_variant(V2, name="aa_fp6_paged", batch=3, q_tokens=2, kv_len=0, lengths=(100, 520, 64),
                  kv_dtype="fp6", layout="paged"),
    small_variant(V2, name="aa_lite_n16_paged", batch=4, n_heads=16, kv_len=0,
                  lengths=(1, 33, 700, 64), layout="paged"),
    WORKLOADS["tiny_fp32"],
], ids=lambda w: w.name)
def test_absorb_append_matches_separate_calls(w):
    """mla_absorb_append (one launch on the fast paths, two otherwise) writes
    the same bytes as mla_absorb_q followed by mla_cache_append: the absorbed
    query and every cache byte and scale, with cache and query pre-filled
    with a byte pattern so that only the step's new rows are written."""
    say(f"case absorb_append {w.name}: B={w.batch} T={w.q_tokens} kv={w.kv_dtype} layout={w.layout}")
    gen = generate(w)
    bufs = [_buffers(w, gen), _buffers(w, gen)]
    for buf in bufs:
        buf.q_abs.view(torch.uint8).fill_(0x5A)
        buf.caches[0].view(torch.uint8).fill_(0x5A)
        if buf.scales[0] is not None:
            buf.scales[0].fill_(0.5)
    bufs[0].absorb()
    bufs[0].append()
    bufs[1].absorb_append()
    torch.cuda.synchronize()
    a, b = bufs
    assert torch.equal(a.q_abs.view(torch.uint8), b.q_abs.view(torch.uint8)), "absorbed query"
    assert torch.equal(a.caches[0].view(torch.uint8), b.caches[0].view(torch.uint8)), "cache"
    assert not torch.equal(a.caches[0].view(torch.uint8),
                           torch.full_like(a.caches[0].view(torch.uint8), 0x5A)), "rows written"
    if a.scales[0] is not None:
        assert torch.equal(a.scales[0], b.scales[0]), "scales"
