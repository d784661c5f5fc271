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
(they must match decode_mfma.hip, decode_fp8.hip and decode_x2.hip: LROW is
also the row pitch of the split-operand kernel's tiles):
python3 gen_decode_asm.py
"""
LROW = 1168          # LDS bytes per bf16 token row (also decode_x2.hip)
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


def pvd(with_softmax=False, with_dma=False):
    """PV product of one tile for this wave's 128 latent dims and all 128
    query rows of the workgroup: O^T[dims, rows] += C^T[dims, tok] P^T[tok,
    rows], 32 MFMAs (4 dim blocks x 4 row blocks x 2 token halves).  The
    weights of every row block come from the LDS P buffer (written there by
    the waves that own the rows); each weight fragment is read once and used
    for 4 MFMAs, each transposed C^T fragment read once and used for 4.
    with_softmax: the softmax of the current tile is interleaved (two vector
    instructions per MFMA).

    operands: %0..%15 O blocks (block 4 db + rb: dims 32 db of the wave's
    128, rows 32 rb), %16..%31 the current tile's scores s_0..s_15 (in;
    overwritten), %32..%39 its packed bf16 weight pairs (out), %40 its
    scaled max (out), %41 a temporary, %42 the running normaliser (in/out),
    %43 base address of this lane's transposed reads (slot of the previous
    tile + the wave's dim offset), %44 this lane's P fragment address, %45
    -m_ref, %46 the scale (log2 domain).  with_dma: %47 buffer descriptor,
    %48 LDS base of this wave's loads, %49..%52 lane offsets of loads 5..8.
    Without the softmax only %0..%15, %16 (= transposed-read base) and %17
    (= P fragment address) are used.
    Fixed registers: P fragments v[224:255], C^T fragment buffers
    v[PVD_VBUF:223].
    """
    vbase, pbase = ("%43", "%44") if with_softmax else ("%16", "%17")
    valu = []
    if with_softmax:
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
        return 224 + 4 * (4 * ks + rb)

    def vbuf(g):
        return PVD_VBUF + 4 * (g % PVD_NVBUF)

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

    for rb in range(4):
        pread(rb, 0)
    for g in range(PVD_AHEAD):
        vread(g)
    for rb in range(4):
        pread(rb, 1)
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
        if with_dma and i % 8 == 3 and i // 8 < PV_DMA:
            k = i // 8
            out += dma(QK_DMA + k, "%47", "%48", f"%{49 + k}")
        take = 2 if i < 31 else len(valu) - vi
        for _ in range(take):
            if vi < len(valu):
                out.append(valu[vi])
                vi += 1
    assert vi == len(valu)
    return out


# ---------------------------------------------------------------- fp8 tiles
# The fp8 kernel (decode_fp8.hip) keeps raw E4M3 tiles in LDS (rows of 576
# codes at a pitch of LROW8 bytes) and converts the MFMA operands in
# registers with v_cvt_scalef32_pk_bf16_fp8 (two codes per instruction, exact:
# every E4M3 value is a bf16 value).  A vector write needs two wait states
# before a matrix instruction reads it as an operand; the sequences keep at
# least that many instructions in between.
LROW8 = 592          # LDS bytes per fp8 token row (576 + 16 pad)
QK8_AHEAD = 3        # raw 16-byte reads in flight ahead of the current pair
QK8_DMA = 4          # tile loads interleaved with the score sequence
QK8_RAW = 224        # 4 raw read buffers v[224:239]
QK8_CVT = 240        # 4 converted operand buffers v[240:255]
PV8_P = 240          # P fragments v[240:255]
PV8_CVT = 232        # 2 converted C^T fragment buffers v[232:239]
PV8_RAW = 226        # 3 raw C^T fragment buffers v[226:231]
PV8_KV = 210         # the tile's 16 token scales v[210:225] (with the softmax)


def cvt8(dst, src, hi):
    sel = " op_sel:[1,0,0]" if hi else ""
    return f"v_cvt_scalef32_pk_bf16_fp8 v{dst}, v{src}, 1.0{sel}"


def qk8(with_dma=True):
    """Scores of one raw fp8 tile for the wave's 32 query rows: S^T[tok, row]
    = K Q^T, 36 MFMAs in pairs.  Lane l reads 16 codes of token row l%32 at
    dims 32kk + 16(l/32) (one ds_read_b128 per pair kk); the first 8 become
    the A operand of MFMA 2kk, the last 8 that of MFMA 2kk+1, so MFMA 2kk
    takes dims {32kk + 0..7, 32kk + 16..23} and MFMA 2kk+1 the others (the
    query fragments are laid out to match).  The pair kk+1 is converted
    while the pair kk runs.

    operands: %0 S (floatx16, out), %1 base address of this lane's reads,
    %2..%37 query fragments, %38 buffer descriptor of the tile being loaded,
    %39 LDS base of this wave's loads of it, %40..%43 lane offsets of its
    loads 0..3 (one after every fourth MFMA pair)."""
    out, issued = [], []
    npair = 18

    def raw(kk):
        return QK8_RAW + 4 * (kk % 4)

    def conv(i):
        return QK8_CVT + 4 * (i % 4)

    def read(kk):
        r = raw(kk)
        out.append(f"ds_read_b128 v[{r}:{r + 3}], %1 offset:{32 * kk}")
        issued.append(kk)

    def wait(kk):
        last = issued.index(kk)
        out.append(f"s_waitcnt lgkmcnt({min(15, len(issued) - 1 - last)})")

    def convert(kk, half):
        r, c = raw(kk), conv(2 * kk + half)
        return [cvt8(c, r + 2 * half, False), cvt8(c + 1, r + 2 * half, True),
                cvt8(c + 2, r + 2 * half + 1, False), cvt8(c + 3, r + 2 * half + 1, True)]

    for kk in range(QK8_AHEAD):
        read(kk)
    wait(0)
    out += convert(0, 0) + convert(0, 1)
    for kk in range(npair):
        if kk + QK8_AHEAD < npair:
            read(kk + QK8_AHEAD)
        for half in range(2):
            i = 2 * kk + half
            c = "0" if i == 0 else "%0"
            out.append(f"v_mfma_f32_32x32x16_bf16 %0, v[{conv(i)}:{conv(i) + 3}], %{2 + i}, {c}")
            if kk + 1 < npair:
                if half == 0:
                    wait(kk + 1)
                out += convert(kk + 1, half)
        if with_dma and kk % 4 == 1 and kk // 4 < QK8_DMA:
            n = kk // 4
            out += dma(n, "%38", "%39", f"%{40 + n}")
    return out


def softmax8_valu(S, KV, TMP, LRUN, NEGM, SCALE, PWADDR):
    """Softmax of one fp8 tile: the raw scores times their token scales, p_r
    = 2^(s_r * scale - m_ref) against the row's fixed reference (no max:
    overflow is checked once per pass, on the normaliser).  The normaliser
    sums the bf16-rounded p_r (pairs packed in place, then two interleaved
    dot products with (1, 1) into LRUN and TMP).  The PV weights p_r times
    the token scale (the cache codes enter the MFMA unscaled) go into the
    scale registers, are packed to bf16 pairs in place (KV(0..7)) and
    written to this wave's P fragments at PWADDR (token halves 0 and 1).
    Each v_exp result is read at least two instructions later."""
    fma = [f"v_fma_f32 {S(r)}, {S(r)}, {SCALE}, {NEGM}" for r in range(16)]
    exp = [f"v_exp_f32 {S(r)}, {S(r)}" for r in range(16)]
    seq = [f"v_mul_f32 {S(r)}, {S(r)}, {KV(r)}" for r in range(16)]
    seq += fma[:2]
    for r in range(2, 16):
        seq += [fma[r], exp[r - 2]]
    seq += exp[14:]
    seq += [f"v_mov_b32 {TMP}, 0", "s_nop 1"]
    seq += [f"v_mul_f32 {KV(r)}, {S(r)}, {KV(r)}" for r in range(16)]
    seq += [f"v_cvt_pk_bf16_f32 {S(i)}, {S(2 * i)}, {S(2 * i + 1)}" for i in range(8)]
    for j in range(4):
        seq += [f"v_dot2c_f32_bf16 {LRUN}, 0x3f803f80, {S(2 * j)}",
                f"v_dot2c_f32_bf16 {TMP}, 0x3f803f80, {S(2 * j + 1)}"]
    seq += [f"v_cvt_pk_bf16_f32 {KV(i)}, {KV(2 * i)}, {KV(2 * i + 1)}" for i in range(8)]
    seq += [f"v_add_f32 {LRUN}, {LRUN}, {TMP}"]
    k0 = KV(0)[1:]
    seq += [f"ds_write_b128 {PWADDR}, v[{k0}:{int(k0) + 3}]",
            f"ds_write_b128 {PWADDR}, v[{int(k0) + 4}:{int(k0) + 7}] offset:1024"]
    return seq


def pv8(with_softmax=True):
    """PV product of one raw fp8 tile for this wave's 128 latent dims and
    all 128 rows: O^T[dims, rows] += C^T[dims, tok] P^T[tok, rows], 32 MFMAs
    (4 dim blocks x 4 row blocks x 2 token halves).  C^T fragment (ks, db)
    comes from one ds_read_b64_tr_b8 per lane (8 codes: one latent dim of 8
    tokens) and 4 conversions; it feeds 4 MFMAs.  The weight fragments of
    all row blocks come from the LDS P buffer of the previous tile.

    with_softmax: the softmax of the current tile (softmax8_valu) is
    interleaved, front-loaded so that its weight writes leave the LDS queue
    before the sequence ends.  operands: %0..%15 O blocks (block 4 db +
    rb), %16..%31 the current tile's raw scores (in; clobbered), %32 a
    temporary, %33 the running normaliser (in/out), %34 this lane's C^T
    read address (slot of the previous tile + lane offset), %35 this lane's
    P fragment address (previous tile's P buffer), %36 the address of this
    lane's 16 token scales (read into v[210:225]), %37 -m_ref, %38 the
    scale (log2 domain), %39 a scalar flag: nonzero zeroes the O blocks
    first (one MFMA of zero operands and a zero accumulator input per
    block, skipped by a branch inside the sequence otherwise), %40 this
    lane's address in the P buffer of the current tile.
    Without the softmax: %0..%15, %16 the C^T address, %17 the P address."""
    if with_softmax:
        kv = lambda r: f"v{PV8_KV + r}"
        valu = softmax8_valu(lambda r: f"%{16 + r}", kv, "%32", "%33", "%37", "%38", "%40")
        vaddr, paddr = "%34", "%35"
    else:
        valu = []
        vaddr, paddr = "%16", "%17"
    out, issued = [], []

    def read(name, instr):
        out.append(instr)
        issued.append(name)

    def wait_for(names):
        last = max(i for i, n in enumerate(issued) if n in names)
        out.append(f"s_waitcnt lgkmcnt({min(15, len(issued) - 1 - last)})")

    def raw(g):
        return PV8_RAW + 2 * (g % 3)

    def conv(g):
        return PV8_CVT + 4 * (g % 2)

    def vread(g):
        ks, db = g // 4, g % 4
        read(("V", g), f"ds_read_b64_tr_b8 v[{raw(g)}:{raw(g) + 1}], {vaddr} "
                       f"offset:{16 * LROW8 * ks + 32 * db}")

    def pread(rb, ks):
        r = PV8_P + 4 * rb
        read(("P", rb, ks), f"ds_read_b128 v[{r}:{r + 3}], {paddr} offset:{1024 * (2 * rb + ks)}")

    def convert(g):
        r, c = raw(g), conv(g)
        return [cvt8(c, r, False), cvt8(c + 1, r, True), cvt8(c + 2, r + 1, False),
                cvt8(c + 3, r + 1, True)]

    if with_softmax:
        z = PV8_P + 12
        out += ["s_cmp_eq_u32 %39, 0", "s_cbranch_scc1 MLA_PV8_NZ%=",
                f"v_mov_b32 v{z}, 0", f"v_mov_b32 v{z + 1}, 0", f"v_mov_b32 v{z + 2}, 0",
                f"v_mov_b32 v{z + 3}, 0", "s_nop 1"]
        out += [f"v_mfma_f32_32x32x16_bf16 %{i}, v[{z}:{z + 3}], v[{z}:{z + 3}], 0"
                for i in range(16)]
        out += ["s_nop 7", "s_nop 7", "MLA_PV8_NZ%=:"]
        for q in range(4):
            read("K", f"ds_read_b128 v[{PV8_KV + 4 * q}:{PV8_KV + 4 * q + 3}], %36 offset:{16 * q}")
    vread(0)
    for rb in range(4):
        pread(rb, 0)
    vread(1)
    vread(2)
    vi = 0
    if with_softmax:
        wait_for({"K"})                       # the scales, before the first scaling
    def put_valu():
        nonlocal vi
        x = valu[vi]
        vi += 1
        if x.startswith("ds_write"):
            read(("W", vi), x)                # counted by lgkmcnt like the reads
        else:
            out.append(x)

    for _ in range(6):                        # independent softmax work first
        if vi < len(valu):
            put_valu()
    wait_for({("V", 0)})
    out += convert(0)
    for i in range(32):
        ks, db, rb = i // 16, (i // 4) % 4, i % 4
        g = i // 4
        if rb == 0:
            wait_for({("P", rr, ks) for rr in range(4)} if i in (0, 16) else {("V", g)})
        out.append(f"v_mfma_f32_32x32x16_bf16 %{4 * db + rb}, v[{conv(g)}:{conv(g) + 3}], "
                   f"v[{PV8_P + 4 * rb}:{PV8_P + 4 * rb + 3}], %{4 * db + rb}")
        if 12 <= i < 16:
            pread(i - 12, 1)                  # after the last use of P(rb, 0)
        if rb == 1 and g + 1 < 8:
            wait_for({("V", g + 1)})
            out += convert(g + 1)             # read by MFMA 4(g+1), >= 2 instructions later
        if rb == 2 and g + 3 < 8:
            vread(g + 3)                      # into the buffer of fragment g, converted already
        take = 4 if i < 31 else len(valu) - vi
        for _ in range(take):
            if vi < len(valu):
                put_valu()
    assert vi == len(valu)
    return out


PV8_S = 194          # the current tile's scores v[194:209] (fused step only)


def step8():
    """A whole steady-state step of the fp8 kernel as one sequence: the
    scores of tile it (as qk8, into the fixed registers v[194:209]), then the
    PV product of tile it-1 with the softmax of tile it interleaved (as pv8).
    Being one sequence lets the PV product's first operand reads go out
    while the last score MFMAs run, each into a buffer whose last reader has
    been issued: the token scales and C^T fragment 0 once the raw buffer of
    score pair 16 is converted, fragments 1 and 2 once that of pair 17 is,
    and weight fragment rb right after score MFMA 32 + rb, the last reader
    of its register quad.  The PV MFMAs then follow the score MFMAs with no
    LDS round trip in between.  For tiles with no masked token after the
    first one (the row references are set); the others take the two
    sequences with the kernel's masking code between them.

    operands: %0..%15 O blocks (block 4 db + rb), %16 the running
    normaliser (in/out), %17 a temporary, %18 base address of this lane's
    score reads (slot of tile it), %19..%54 query fragments, %55 buffer
    descriptor of the tile being loaded, %56 LDS base of this wave's loads
    of it, %57..%60 lane offsets of its loads 0..3, %61 this lane's C^T read
    address (slot of tile it-1), %62 this lane's P fragment address (buffer
    of tile it-1), %63 the address of this lane's 16 token scales of tile
    it, %64 -m_ref, %65 the scale (log2 domain), %66 this lane's address in
    the P buffer of tile it."""
    S = lambda r: f"v{PV8_S + r}"
    kv = lambda r: f"v{PV8_KV + r}"
    valu = softmax8_valu(S, kv, "%17", "%16", "%64", "%65", "%66")
    sreg = f"v[{PV8_S}:{PV8_S + 15}]"
    out, issued = [], []

    def read(name, instr):
        out.append(instr)
        issued.append(name)

    def wait_for(names):
        last = max(i for i, n in enumerate(issued) if n in names)
        out.append(f"s_waitcnt lgkmcnt({min(15, len(issued) - 1 - last)})")

    # ---- scores (qk8 with the PV prologue reads hoisted into its tail)
    def qraw(kk):
        return QK8_RAW + 4 * (kk % 4)

    def qconv(i):
        return QK8_CVT + 4 * (i % 4)

    def qread(kk):
        r = qraw(kk)
        read(("Q", kk), f"ds_read_b128 v[{r}:{r + 3}], %18 offset:{32 * kk}")

    def qconvert(kk, half):
        r, c = qraw(kk), qconv(2 * kk + half)
        return [cvt8(c, r + 2 * half, False), cvt8(c + 1, r + 2 * half, True),
                cvt8(c + 2, r + 2 * half + 1, False), cvt8(c + 3, r + 2 * half + 1, True)]

    def vraw(g):
        return PV8_RAW + 2 * (g % 3)

    def vconv(g):
        return PV8_CVT + 4 * (g % 2)

    def vread(g):
        ks, db = g // 4, g % 4
        read(("V", g), f"ds_read_b64_tr_b8 v[{vraw(g)}:{vraw(g) + 1}], %61 "
                       f"offset:{16 * LROW8 * ks + 32 * db}")

    def pread(rb, ks):
        r = PV8_P + 4 * rb
        read(("P", rb, ks), f"ds_read_b128 v[{r}:{r + 3}], %62 offset:{1024 * (2 * rb + ks)}")

    def vconvert(g):
        r, c = vraw(g), vconv(g)
        return [cvt8(c, r, False), cvt8(c + 1, r, True), cvt8(c + 2, r + 1, False),
                cvt8(c + 3, r + 1, True)]

    npair = 18
    for kk in range(QK8_AHEAD):
        qread(kk)
    wait_for({("Q", 0)})
    out += qconvert(0, 0) + qconvert(0, 1)
    for kk in range(npair):
        if kk + QK8_AHEAD < npair:
            qread(kk + QK8_AHEAD)
        for half in range(2):
            i = 2 * kk + half
            c = "0" if i == 0 else sreg
            out.append(f"v_mfma_f32_32x32x16_bf16 {sreg}, v[{qconv(i)}:{qconv(i) + 3}], "
                       f"%{19 + i}, {c}")
            if kk + 1 < npair:
                if half == 0:
                    wait_for({("Q", kk + 1)})
                out += qconvert(kk + 1, half)
            if i >= 32:
                pread(i - 32, 0)              # its quad's last reader (MFMA i) is issued
            if i == 31:                       # raw quads of pairs 14..16 are converted
                for q in range(4):
                    read("K", f"ds_read_b128 v[{PV8_KV + 4 * q}:{PV8_KV + 4 * q + 3}], "
                              f"%63 offset:{16 * q}")
                vread(0)
            if i == 33:                       # ... and that of pair 17
                vread(1)
                vread(2)
        if kk % 4 == 1 and kk // 4 < QK8_DMA:
            n = kk // 4
            out += dma(n, "%55", "%56", f"%{57 + n}")

    # ---- PV product of tile it-1 with the softmax of tile it
    vi = 0

    def put_valu():
        nonlocal vi
        x = valu[vi]
        vi += 1
        if x.startswith("ds_write"):
            read(("W", vi), x)                # counted by lgkmcnt like the reads
        else:
            out.append(x)

    wait_for({("V", 0)})
    out += vconvert(0)
    for i in range(32):
        ks, db, rb = i // 16, (i // 4) % 4, i % 4
        g = i // 4
        if i < 4 or 16 <= i < 20:
            wait_for({("P", rb, ks)})
        elif rb == 0:
            wait_for({("V", g)})
        out.append(f"v_mfma_f32_32x32x16_bf16 %{4 * db + rb}, v[{vconv(g)}:{vconv(g) + 3}], "
                   f"v[{PV8_P + 4 * rb}:{PV8_P + 4 * rb + 3}], %{4 * db + rb}")
        if 12 <= i < 16:
            pread(i - 12, 1)                  # after the last use of P(rb, 0)
        if rb == 1 and g + 1 < 8:
            wait_for({("V", g + 1)})
            out += vconvert(g + 1)            # read by MFMA 4(g+1), >= 2 instructions later
        if rb == 2 and g + 3 < 8:
            vread(g + 3)                      # into the buffer of fragment g, converted already
        if i == 1:
            # the scores' last MFMA ended before PV MFMA 1 started; the
            # nops cover the matrix-result-to-vector-read distance besides
            out.append("s_nop 7")
            out.append("s_nop 7")
            wait_for({"K"})
        if i >= 1:
            take = 4 if i < 31 else len(valu) - vi
            for _ in range(take):
                if vi < len(valu):
                    put_valu()
    assert vi == len(valu)
    return out


# ------------------------------------------------------ split-operand scores
X2_AHEAD = 5         # tile-operand reads in flight ahead of the current pair
X2_RAW = 232         # 6 read buffers v[232:255]


def qkx2():
    """Scores of one bf16 tile for a split-operand wave's 16 query rows:
    S^T[tok, row] = K (Q_hi + Q_lo)^T with v_mfma_f32_16x16x32_bf16, tokens
    as M in two blocks of 16, the hi and lo parts of the query in separate
    accumulators (4 in all).  Read n (n = 2 ks + tb) fetches the 8 dims
    32 ks + 8 (l/16) .. +7 of this lane's token row of block tb and feeds the
    hi and the lo MFMA of (ks, tb); five reads stay in flight ahead.

    operands: %0 %1 S_hi of token blocks 0 and 1, %2 %3 S_lo (floatx4, out),
    %4 base address of this lane's reads (token block 0, dim group l/16),
    %5..%22 Q_hi fragments (ks = 0..17), %23..%40 Q_lo fragments."""
    out, issued = [], []
    nbuf = X2_AHEAD + 1

    def buf(n):
        return X2_RAW + 4 * (n % nbuf)

    def read(n):
        ks, tb = n // 2, n % 2
        r = buf(n)
        out.append(f"ds_read_b128 v[{r}:{r + 3}], %4 offset:{16 * LROW * tb + 64 * ks}")
        issued.append(n)

    def wait(n):
        out.append(f"s_waitcnt lgkmcnt({min(15, len(issued) - 1 - issued.index(n))})")

    nread = 2 * (QK_STEPS // 2)
    for n in range(X2_AHEAD):
        read(n)
    for n in range(nread):
        ks, tb = n // 2, n % 2
        wait(n)
        r = buf(n)
        for part, (acc, q) in enumerate(((tb, 5 + ks), (2 + tb, 23 + ks))):
            c = "0" if ks == 0 else f"%{acc}"
            out.append(f"v_mfma_f32_16x16x32_bf16 %{acc}, v[{r}:{r + 3}], %{q}, {c}")
        if n + X2_AHEAD < nread:
            read(n + X2_AHEAD)                # into the buffer of read n-1, consumed
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
    txt.append(emit("MLA_ASM_PVD_SOFTMAX_TILE", pvd(True, False)))
    txt.append(f"#define MLA_ASM_PVD_CLOBBERS {clobbers(PVD_VBUF, 256 - PVD_VBUF)}\n")
    txt.append(emit_plain("MLA_ASM_SOFTMAX_MAX", softmax_max()))
    txt.append(emit("MLA_ASM_QK8_TILE", qk8()))
    txt.append(f"#define MLA_ASM_QK8_CLOBBERS {clobbers(QK8_RAW, 32)}\n")
    txt.append(emit("MLA_ASM_PV8_SOFTMAX_TILE", pv8(True)))
    txt.append(emit("MLA_ASM_PV8_TILE", pv8(False)))
    txt.append(f"#define MLA_ASM_PV8_CLOBBERS {clobbers(PV8_RAW, 256 - PV8_RAW)}\n")
    txt.append(f"#define MLA_ASM_PV8_SOFTMAX_CLOBBERS {clobbers(PV8_KV, 256 - PV8_KV)}\n")
    txt.append(emit("MLA_ASM_STEP8_TILE", step8()))
    txt.append(emit("MLA_ASM_QKX2_TILE", qkx2()))
    txt.append(f"#define MLA_ASM_QKX2_CLOBBERS {clobbers(X2_RAW, 256 - X2_RAW)}\n")
    txt.append(f"#define MLA_ASM_STEP8_CLOBBERS {clobbers(PV8_S, 256 - PV8_S)}\n")

    open("decode_mfma_asm.inc", "w").write("\n".join(txt))
