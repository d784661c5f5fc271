#!/usr/bin/env python3
"""Writes decode_mfma_asm.inc: the software-pipelined LDS-read / MFMA
sequences of the attention kernel's tile steps, as inline-assembly string
literals.

The compiler keeps a single LDS operand read in flight in front of each
matrix instruction; these sequences keep several in flight (the reads of the
next P instructions are issued before waiting for the current one), so the
LDS latency hides behind the matrix pipe.  The softmax of a tile is
interleaved with the PV product of the previous tile, and the loads of the
tile after next are spread through both sequences, so the vector ALU and the
memory pipeline work while the matrix pipe runs.  Each sequence waits for
all of its own LDS reads before it ends (its buffer loads complete into LDS
and are waited for by the kernel) and finishes with enough independent
cycles for a vector instruction to read the matrix results.

Run from this directory after changing the tile layout constants below
(they must match decode_mfma.hip):  python3 gen_decode_asm.py
"""
LROW = 1168          # LDS bytes per token row
QK_STEPS = 36        # 576 / 16 dims per v_mfma_f32_32x32x16_bf16
QK_AHEAD = 6         # reads in flight ahead of the current MFMA
QK_BUFS = 8
PVD_AHEAD = 2        # C^T fragments read ahead (each feeds 4 MFMAs)
PVD_NVBUF = 4        # C^T fragment buffers
PVD_LEAD = 8         # softmax instructions before the first PV MFMA
QK_DMA = 5           # tile loads interleaved with the QK sequence
PV_DMA = 4           # ... and with the PV + softmax sequence (9 per wave)
NOPS = "s_nop 7\\n\\ts_nop 7\\n\\t"   # 16 wait states: XDL result -> VALU read


QK_TMP = 224         # first VGPR of the QK operand buffers (8 x 4)
PVD_VBUF = 224 - 4 * PVD_NVBUF   # first VGPR of the C^T fragment buffers


def quad(base, i, nbuf):
    r = base + 4 * (i % nbuf)
    return r


def dma(n, rsrc, ldsbase, voff):
    """Load n of this wave's share of a tile: 64 lanes x 16 bytes from the
    cache (buffer descriptor rsrc, lane offset voff) straight into LDS at
    ldsbase + 4096 n (M0 holds the LDS address)."""
    return [f"s_add_u32 m0, {ldsbase}, {4096 * n}", "s_nop 0",
            f"buffer_load_dwordx4 {voff}, {rsrc}, 0 offen lds"]


def qk(with_dma=False):
    # operands: %0 S (floatx16, out), %1 base address, %2..%37 query
    # fragments; with_dma: %38 buffer descriptor, %39 LDS base of this
    # wave's loads, %40..%44 lane offsets of loads 0..4 (one load after
    # every fourth MFMA).  Operand buffers are the fixed VGPRs v[224:255].
    out = []
    for k in range(QK_AHEAD):
        r = quad(QK_TMP, k, QK_BUFS)
        out.append(f"ds_read_b128 v[{r}:{r + 3}], %1 offset:{32 * k}")
    for k in range(QK_STEPS):
        n = k + QK_AHEAD
        if n < QK_STEPS:
            r = quad(QK_TMP, n, QK_BUFS)
            out.append(f"ds_read_b128 v[{r}:{r + 3}], %1 offset:{32 * n}")
        out.append(f"s_waitcnt lgkmcnt({min(QK_AHEAD, QK_STEPS - 1 - k)})")
        c = "0" if k == 0 else "%0"
        r = quad(QK_TMP, k, QK_BUFS)
        out.append(f"v_mfma_f32_32x32x16_bf16 %0, v[{r}:{r + 3}], %{2 + k}, {c}")
        if with_dma and k % 4 == 3 and k // 4 < QK_DMA:
            n = k // 4
            out += dma(n, "%38", "%39", f"%{40 + n}")
    return out


def max_valu(S, MT, TMP, SCALE):
    """Scaled max of the 16 raw scores and of the lane pair (l, l ^ 32).
    v_permlane32_swap exchanges the upper half of its first operand with
    the lower half of its second: with the max in both, the larger of the
    two results is the pair's max."""
    valu = [f"v_max3_f32 {TMP}, {S(0)}, {S(1)}, {S(2)}"]
    for r in range(3, 15, 2):
        valu.append(f"v_max3_f32 {TMP}, {TMP}, {S(r)}, {S(r + 1)}")
    valu.append(f"v_max_f32 {TMP}, {TMP}, {S(15)}")
    valu.append(f"v_mov_b32 {MT}, {TMP}")
    valu.append("s_nop 1")
    valu.append(f"v_permlane32_swap_b32 {TMP}, {MT}")
    valu.append("s_nop 1")
    valu.append(f"v_max_f32 {TMP}, {TMP}, {MT}")
    valu.append(f"v_mul_f32 {MT}, {TMP}, {SCALE}")
    return valu


def weights_valu(S, PK, LRUN, NEGM, SCALE):
    """p_r = 2^(s_r * scale - m_ref) (one fma, no rounding in between);
    pairs packed to bf16; normaliser += both rounded weights of each pair.
    Each v_exp result is read at least two instructions later."""
    fma = [f"v_fma_f32 {S(r)}, {S(r)}, {SCALE}, {NEGM}" for r in range(16)]
    exp = [f"v_exp_f32 {S(r)}, {S(r)}" for r in range(16)]
    seq = fma[:2]
    for r in range(2, 16):
        seq += [fma[r], exp[r - 2]]
    seq += exp[14:]
    seq.append("s_nop 1")
    seq += [f"v_cvt_pk_bf16_f32 {PK(i)}, {S(2 * i)}, {S(2 * i + 1)}" for i in range(8)]
    seq += [f"v_dot2c_f32_bf16 {LRUN}, 0x3f803f80, {PK(i)}" for i in range(8)]
    return seq


def weights_valu_fp8(S, PK, LRUN, NEGM, SCALE, KV):
    """fp8 cache: the scores arrive multiplied by their token's scale.  p_r
    as for bf16; the normaliser sums the rounded unscaled weights, and the PV
    weights are p_r times the token scale (the cache values enter the MFMA
    unscaled), packed to bf16."""
    seq = weights_valu(S, PK, LRUN, NEGM, SCALE)
    seq += [f"v_mul_f32 {S(r)}, {S(r)}, {KV(r)}" for r in range(16)]
    seq.append("s_nop 1")
    seq += [f"v_cvt_pk_bf16_f32 {PK(i)}, {S(2 * i)}, {S(2 * i + 1)}" for i in range(8)]
    return seq


def softmax_max():
    """operands: %0 scaled max (out), %1 a temporary, %2..%17 scores, %18 scale."""
    return max_valu(lambda r: f"%{2 + r}", "%0", "%1", "%18") + ["s_nop 1"]


def softmax_valu(S, PK, MT, TMP, LRUN, NEGM, SCALE):
    """One tile's softmax (bf16 weights).  The weights need only the fixed
    reference, not this tile's max, so the max (for the restart check) and
    the weights are independent chains."""
    return max_valu(S, MT, TMP, SCALE) + weights_valu(S, PK, LRUN, NEGM, SCALE)


def pvd(with_softmax=False, with_dma=False, fp8=False):
    """PV product of one tile for this wave's 128 latent dims and all 128
    query rows of the workgroup: O^T[dims, rows] += C^T[dims, tok] P^T[tok,
    rows], 32 MFMAs (4 dim blocks x 4 row blocks x 2 token halves).  The
    weights of every row block come from the LDS P buffer (written there by
    the waves that own the rows); each weight fragment is read once and used
    for 4 MFMAs, each transposed C^T fragment read once and used for 4.
    with_softmax: the softmax of the current tile is interleaved (two vector
    instructions per MFMA, four for the longer fp8 softmax).

    operands: %0..%15 O blocks (block 4 db + rb: dims 32 db of the wave's
    128, rows 32 rb), %16..%31 the current tile's scores s_0..s_15 (in;
    overwritten), %32..%39 its packed bf16 weight pairs (out), %40 its
    scaled max (out), %41 a temporary, %42 the running normaliser (in/out),
    %43 base address of this lane's transposed reads (slot of the previous
    tile + the wave's dim offset), %44 this lane's P fragment address, %45
    -m_ref, %46 the scale (log2 domain).  with_dma: %47 buffer descriptor,
    %48 LDS base of this wave's loads, %49..%52 lane offsets of loads 5..8.
    fp8 (no loads): %16..%31 are the raw scores; %47 is the address of this
    lane's 16 token scales in LDS (read into v[212:227]); the sequence
    multiplies the scores by them first.
    Without the softmax only %0..%15, %16 (= transposed-read base) and %17
    (= P fragment address) are used.
    Fixed registers: P fragments v[224:255], C^T fragment buffers
    v[PVD_VBUF:223].  fp8 (which also holds the staged next tile): P
    fragments v[240:255], the second token half's fragments read into them 4
    MFMAs after the first half's last use, 3 C^T buffers v[228:239], token
    scales v[212:227].
    """
    vbase, pbase = ("%43", "%44") if with_softmax else ("%16", "%17")
    valu = []
    if with_softmax and fp8:
        kv = lambda r: f"v{212 + r}"
        valu = ([f"v_mul_f32 %{16 + r}, %{16 + r}, {kv(r)}" for r in range(16)]
                + max_valu(lambda r: f"%{16 + r}", "%40", "%41", "%46")
                + weights_valu_fp8(lambda r: f"%{16 + r}", lambda i: f"%{32 + i}",
                                   "%42", "%45", "%46", kv))
    elif with_softmax:
        valu = softmax_valu(lambda r: f"%{16 + r}", lambda i: f"%{32 + i}",
                            "%40", "%41", "%42", "%45", "%46")
    out, issued = [], []

    def read(name, instrs):
        for x in instrs:
            out.append(x)
            issued.append(name)

    def wait_for(names):
        last = max(i for i, n in enumerate(issued) if n in names)
        out.append(f"s_waitcnt lgkmcnt({min(15, len(issued) - 1 - last)})")

    def pfrag(rb, ks):
        return 240 + 4 * rb if fp8 else 224 + 4 * (4 * ks + rb)

    def vbuf(g):
        return (228 + 4 * (g % 3)) if fp8 else PVD_VBUF + 4 * (g % PVD_NVBUF)

    def vread(g):
        ks, db = g // 4, g % 4
        r = vbuf(g)
        lo = (16 * ks) * LROW + 64 * db
        hi = (16 * ks + 2) * LROW + 64 * db
        read(("V", g), [f"ds_read_b64_tr_b16 v[{r}:{r + 1}], {vbase} offset:{lo}",
                        f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], {vbase} offset:{hi}"])

    def pread(rb, ks):
        r = pfrag(rb, ks)
        read(("P", rb, ks), [f"ds_read_b128 v[{r}:{r + 3}], {pbase} offset:{1024 * (2 * rb + ks)}"])

    if fp8 and with_softmax:
        for q in range(4):
            read("K", [f"ds_read_b128 v[{212 + 4 * q}:{215 + 4 * q}], %47 offset:{16 * q}"])
    for rb in range(4):
        pread(rb, 0)
    for g in range(PVD_AHEAD):
        vread(g)
    if not fp8:
        for rb in range(4):
            pread(rb, 1)
    if fp8 and with_softmax:
        wait_for({"K"})                       # the scales, before the first scaling
    vi = 0
    for _ in range(PVD_LEAD):                 # independent softmax work first
        if vi < len(valu):
            out.append(valu[vi])
            vi += 1
    for i in range(32):
        ks, db, rb = i // 16, (i // 4) % 4, i % 4
        g = i // 4
        if i % 4 == 0 and g + PVD_AHEAD < 8:
            vread(g + PVD_AHEAD)
        wait_for({("V", g), ("P", rb, ks)})
        out.append(f"v_mfma_f32_32x32x16_bf16 %{4 * db + rb}, v[{vbuf(g)}:{vbuf(g) + 3}], "
                   f"v[{pfrag(rb, ks)}:{pfrag(rb, ks) + 3}], %{4 * db + rb}")
        if fp8 and 12 <= i < 16:
            pread(i - 12, 1)                  # after the last use of P(rb, 0)
        if with_dma and i % 8 == 3 and i // 8 < PV_DMA:
            k = i // 8
            out += dma(QK_DMA + k, "%47", "%48", f"%{49 + k}")
        take = (4 if fp8 else 2) if i < 31 else len(valu) - vi
        for _ in range(take):
            if vi < len(valu):
                out.append(valu[vi])
                vi += 1
    assert vi == len(valu)
    return out


def clobbers(base, n):
    return ", ".join(f'"v{base + i}"' for i in range(n))


def emit_plain(name, lines):
    return f"#define {name} \\\n" + " \\\n".join(f'  "{l}\\n\\t"' for l in lines) + "\n"


def emit(name, lines):
    return (f"#define {name} \\\n" + " \\\n".join(f'  "{l}\\n\\t"' for l in lines)
            + f' \\\n  "{NOPS}"\n')


if __name__ == "__main__":
    txt = ["// Generated by gen_decode_asm.py -- do not edit by hand.",
           "// Inline-assembly bodies of the attention kernel's tile steps.",
           ""]
    txt.append(emit("MLA_ASM_QK_TILE", qk()))
    txt.append(emit("MLA_ASM_QK_TILE_DMA", qk(True)))
    txt.append(f"#define MLA_ASM_QK_CLOBBERS {clobbers(QK_TMP, 32)}\n")
    txt.append(emit("MLA_ASM_PVD_TILE", pvd()))
    txt.append(emit("MLA_ASM_PVD_SOFTMAX_TILE_DMA", pvd(True, True)))
    txt.append(emit("MLA_ASM_PVD_SOFTMAX_TILE", pvd(True, False, False)))
    txt.append(emit("MLA_ASM_PVD_SOFTMAX_TILE_FP8", pvd(True, False, True)))
    txt.append(f"#define MLA_ASM_PVD_CLOBBERS {clobbers(PVD_VBUF, 256 - PVD_VBUF)}\n")
    txt.append(f"#define MLA_ASM_PVD_FP8_CLOBBERS {clobbers(212, 44)}\n")
    txt.append(emit_plain("MLA_ASM_SOFTMAX_MAX", softmax_max()))
    open("decode_mfma_asm.inc", "w").write("\n".join(txt))
