"""Generator of the segment body of the dense 128-head MLA split kernel (gfx950).

The kernel in mla_h128.hip computes, for one split (segment) of one row and
one block of 128 query heads, the split stage of the split-KV decode on the
FlashMLA issue page "Sparse MLA decode is not batch-invariant ..." (section
"Where it comes from"): scores against the row's latent KV, an online softmax
and the P.V product over the split's tokens, in 32-token tiles.  The whole
segment -- query load, tile streaming, both products, the softmax and the
lazy rescale -- is one hand-scheduled inline-asm block written by this
script: with one wave per SIMD the wave's instruction issue bounds the tile
loop, so every instruction, wait and register is placed here.  The C++ side
(mla_h128.hip) plans the segment and writes the output block.

Numerics are those of the 32-head-per-wave kernel in mla_split_h32.hip:
S^T = K Q^T with v_mfma_f32_32x32x16_bf16 over 36 k-steps in ascending
order; p = 2^(s scale log2(e) - m + 7) rounded to fp16 (RNE) for the
product while the normaliser sums the fp32 p in token order; V converted
from bf16 to fp16 (round toward zero); O^T += V^T P^T with
v_mfma_f32_32x32x16_f16; a lazily moved reference max (moved when a head's
max exceeds it by more than 2^8).  Every order is fixed by the segment's own
token range.  What differs is the schedule:
  * step it computes S^T of tile it+1 and, in the shadows of those MFMAs,
    the exponentials, fp16 P and row sums of tile it, the vote on the
    rescale of tile it and the loads of tile it+3; as its last four MFMAs
    free the K operand slots, the V^T (dt, 1) fragments of tile it are read
    into them and stay in flight across the barrier;
  * PV of tile it runs j-major (each P fragment is read from LDS once per
    wave, into one of four slots, this wave's own fragment straight from
    registers) and carries the row max and reference move of tile it+1, so
    the alphas of tile it+1 are in LDS before the next step starts and the
    vote never waits;
  * hooks are placed by their measured issue cost in an MFMA's shadow
    (ins_cost), at most four vector-ALU units per MFMA;
  * masked rows (past the split's end, or a whole tile whose page is not in
    the pool) are streamed from a valid page and then cleared in LDS, so
    every tile load takes the same scalar-base form.

The same generator writes a second body for sparse (top-k) segments, the
sparse attention of the FlashMLA issue page (section "Where it comes from"):
the kernel first resolves the segment's top-k slots (at most 1024) into an
LDS window, one 32-bit value per slot that, added to a lane's piece offset,
gives the byte offset of that piece in the latent pool (invalid slots point
at pool row 0), plus one row-valid mask per tile.  Each of a tile's nine
loads then reads its lane's window value, adds the piece offset and loads
from the pool base; masks replace the valid-row counts, so masked rows
anywhere in a tile are cleared in LDS and their scores set to -inf.  The
arithmetic is the dense body's, so a sparse segment gives the bits of the
32-head gather kernel.

Registers (one wave per SIMD, 256 VGPRs + 256 AGPRs):
  a0..a255   output block O^T; tile T = 4 dt + g holds dims 32 dt.. of the
             wave's 128 and head tile (g + wave) & 3
  v0..v143   query slice of the wave's 32 heads (36 B operands)
  v144..v175 two score blocks (current tile, next tile); during PV the
             upper half of the current tile's block holds two P^T slots
  v176..v191 V^T fragments (dt, j=0), fp16
  v192..v207 V^T fragments (dt, j=1); during S^T the K operand ring
  v208..v215 two P^T fragment slots; during S^T the vote's alphas
  v216..v223 this wave's fp16 P (j = 0, 1)
  v224..v228 m_ref, l_run, m_sub, two temporaries
  v229..v244 lane offsets and LDS addresses (K, V^T, P, alphas)
  v245..v253 source offsets of the nine tile loads (sparse: the piece
             offset in the low half, 4 x the piece's tile row in the high)
  v254       conversion scratch, v255 block-table window (sparse: lane t
             holds the row-valid mask of tile t)
"""

import os
import sys

# ---------------------------------------------------------------- layout
TOK = 32                 # tokens per tile
ROW = 1152               # bytes per latent row (576 bf16)
TILE = TOK * ROW         # 36864
NBUF = 4
P_OFF = NBUF * TILE      # fp16 P exchange, 8 KB: [ht][j][lane] x 16 B
X_OFF = P_OFF + 8192     # per-head floats [n32][ht] (alpha; l in the epilogue)
LDS_BYTES = X_OFF + 512  # 156160
# sparse segments: window values of up to 1024 slots, then 32 tile masks
WIN_SLOTS = 1024
WIN_OFF = LDS_BYTES
MASK_OFF = WIN_OFF + 4 * WIN_SLOTS
SPARSE_LDS_BYTES = MASK_OFF + 4 * (WIN_SLOTS // 32)   # 160384
KSTEPS = 36
KDEPTH = 4
LOADS = 9                # 16-byte direct loads per wave per tile
NEG_INF = "0xff800000"
RESCALE_THR = "0x41000000"   # 8.0 (log2 units)
P_SHIFT_NEG = "0xc0e00000"   # -7.0
FLOOR = "0xf149f2ca"         # -1e30
HOOK_CAP_QK = 4
HOOK_CAP_PV = 4

# SGPRs owned by the asm block (declared clobbered)
S_IT = "s64"        # tile index of the current step
S_PN = "s65"        # page index of the next tile to stream
S_ON = "s66"        # its offset in the page
S_U0 = "s67"        # its first token
S_PBASE = "s68"     # first page of the block-table window
S_LI = "s69"        # window lane of S_PN
S_NV1, S_NV2, S_NV3 = "s70", "s71", "s72"   # valid rows of tiles it+1, it+2, it+3
S_NV0 = "s81"       # valid rows of tile 0 (prologue only; shares S_T3)
S_VOTE, S_VOTE_LO, S_VOTE_HI = "s[74:75]", "s74", "s75"
S_B, S_B0, S_B1 = "s[76:77]", "s76", "s77"  # source base of the tile being streamed
S_T0, S_T1, S_T2, S_T3 = "s78", "s79", "s80", "s81"
S_M0B = "s82"       # LDS address of this wave's first load of the streamed tile
S_LDSW = "s83"      # LDS base + 1024 wave
S_KB = "s84"        # LDS base of tile it+1
S_M0SAVE = "s85"    # the compiler's M0, restored at the end of the block
S_EXEC = "s[86:87]"
S_WINU = S_PN       # sparse: LDS address of the window values of the tile being planned
S_WINB = S_PBASE    # sparse: LDS address of the window
OWNED_SGPRS = [f"s{i}" for i in range(64, 73)] + [f"s{i}" for i in range(74, 88)]


def Q(kk):
    return f"v[{4 * kk}:{4 * kk + 3}]"


S_BASE = (144, 160)


def S(p):
    return f"v[{S_BASE[p]}:{S_BASE[p] + 15}]"


def Se(p, e):
    return f"v{S_BASE[p] + e}"


V0_BASE, V1_BASE = 176, 192


def V0(dt):
    return f"v[{V0_BASE + 4 * dt}:{V0_BASE + 3 + 4 * dt}]"


def V1(dt):
    return f"v[{V1_BASE + 4 * dt}:{V1_BASE + 3 + 4 * dt}]"


def KR(m):
    return f"v[{192 + 4 * m}:{195 + 4 * m}]"


def PR(s):
    return f"v[{208 + 4 * s}:{211 + 4 * s}]"


def PH(j):
    return f"v[{216 + 4 * j}:{219 + 4 * j}]"


M_REF, L_RUN, M_SUB, T0, T1 = "v224", "v225", "v226", "v227", "v228"
KL0 = "v229"


def KA(m):
    return f"v{230 + m}"


VL0 = "v234"


def VA(m):
    return f"v{235 + m}"


PW = "v239"


def PRG(g):
    return f"v{239 + g}"   # g = 1..3


XW, XR = "v243", "v244"


def LO(i):
    return f"v{245 + i}"


LO_REGS = [LO(i) for i in range(9)]


CV = "v254"
PWIN = "v255"

# row t = p / 72 of piece slot p, as (p * 7282) >> 19, exact for p < 2304
DIV72_MUL, DIV72_SHIFT = 7282, 19
assert all((p * DIV72_MUL) >> DIV72_SHIFT == p // 72 for p in range(2304))


class Emitter:
    """Instruction list with LDS-operation tracking.  A wave's LDS operations
    complete in issue order, so waiting for operation k means waiting until
    at most (issued - k - 1) are outstanding (the field holds up to 15)."""

    def __init__(self):
        self.lines = []
        self.issued = 0
        self.done = 0

    def op(self, text):
        if text.startswith("ds_"):
            return self.lds(text)
        self.lines.append("\t" + text)
        return None

    def lds(self, text):
        self.lines.append("\t" + text)
        idx = self.issued
        self.issued += 1
        return idx

    def wait(self, idx):
        if idx is None or idx < self.done:
            return
        n = min(self.issued - idx - 1, 15)
        self.lines.append(f"\ts_waitcnt lgkmcnt({n})")
        self.done = self.issued - n

    def wait_all(self):
        if self.done < self.issued:
            self.lines.append("\ts_waitcnt lgkmcnt(0)")
        self.done = self.issued

    def reset(self):
        # at a point where every LDS operation is known complete
        self.issued = self.done = 0

    def label(self, name):
        self.lines.append(f"{name}_%=:")

    @staticmethod
    def ref(name):
        return f"{name}_%="

    def comment(self, text):
        self.lines.append(f"\t; {text}")


class Item:
    """A group of instructions placed together in one MFMA shadow.  `deps`
    are (item, min_distance_in_steps); a `wait` is an LDS operation index
    (or a callable giving it) that must be complete before the group."""

    def __init__(self, ins, earliest=0, deps=(), wait=None):
        self.ins = list(ins)
        self.earliest = earliest
        self.deps = list(deps)
        self.wait = wait
        self.step = None
        self.lds_idx = None


TRANSCENDENTAL = ("v_exp_f32", "v_log_f32", "v_rcp_f32", "v_rsq_f32", "v_sqrt_f32")


def ins_cost(text):
    """Issue cost of a hook instruction in the shadow of a 32x32x16 MFMA, in
    units of one vector-ALU instruction.  Measured with one wave per SIMD:
    four vector-ALU instructions after each MFMA of a K stream leave it at
    the MFMA's own rate and every further one adds ~4.5 cycles; a
    transcendental counts twice; a 1 KB LDS write costs 20 cycles or more;
    a vector-ALU result read by the scalar unit stalls the wave; scalar-ALU
    instructions and LDS or vector-memory reads cost next to nothing."""
    op = text.split()[0]
    if op in TRANSCENDENTAL:
        return 2.0
    if op == "v_readlane_b32":
        return 2.0
    if op.startswith("v_"):
        return 1.0
    if op == "ds_write_b128":
        return 4.0
    if op.startswith("ds_write"):
        return 1.5
    if op == "s_nop":
        return (int(text.split()[1]) + 1) / 4.0
    if op.startswith(("ds_read", "global_load", "buffer_load")):
        return 0.25
    return 0.0


def item_cost(it):
    return sum(ins_cost(x) for x in it.ins)


def place(items, n_steps, cap):
    """Greedy placement in list order: each group goes to the first step at
    or after its earliest step and its dependencies' steps plus distance,
    where the step's hook cost (ins_cost) stays within `cap` (a group
    costlier than `cap` takes an otherwise empty step)."""
    load = [0.0] * n_steps
    for it in items:
        c = item_cost(it)
        s = it.earliest
        for d, dist in it.deps:
            assert d.step is not None, "dependency placed after its user"
            s = max(s, d.step + dist)
        while s < n_steps - 1 and load[s] > 0 and load[s] + c > cap:
            s += 1
        s = min(s, n_steps - 1)
        it.step = s
        load[s] += c
    slots = [[] for _ in range(n_steps)]
    for it in items:
        slots[it.step].append(it)
    return slots


def emit_items(em, items):
    for it in items:
        w = it.wait() if callable(it.wait) else it.wait
        em.wait(w)
        for x in it.ins:
            idx = em.op(x)
            if idx is not None:
                it.lds_idx = idx


# ---------------------------------------------------------------- pieces


def conv_groups(base_reg):
    """bf16 -> fp16 in place for v[base..base+3], one group per dword: the low
    value shifted up to an fp32, the high one masked, packed toward zero."""
    out = []
    for i in range(4):
        r = f"v{base_reg + i}"
        out.append([f"v_and_b32 {CV}, 0xffff0000, {r}", f"v_lshlrev_b32 {r}, 16, {r}",
                    f"v_cvt_pkrtz_f16_f32 {r}, {r}, {CV}"])
    return out


def vfrag_read_ins(dst_base, dt, j):
    """The two transposing reads of V^T fragment (dt, j) of the wave's dims."""
    m = 2 * (dt & 1)
    off0 = ROW * 16 * j + 128 * (dt >> 1)
    off1 = ROW * (16 * j + 8) + 128 * (dt >> 1)
    return [f"ds_read_b64_tr_b16 v[{dst_base}:{dst_base + 1}], {VA(m)} offset:{off0}",
            f"ds_read_b64_tr_b16 v[{dst_base + 2}:{dst_base + 3}], {VA(m + 1)} offset:{off1}"]


def set_va_ins(sbase):
    """V^T read addresses of the tile whose LDS base is in SGPR sbase (VL0
    already holds the lane offset plus 256 wave)."""
    return [f"v_add_u32 {VA(0)}, {sbase}, {VL0}", f"v_xor_b32 {VA(1)}, 32, {VA(0)}",
            f"v_xor_b32 {VA(2)}, 64, {VA(0)}", f"v_xor_b32 {VA(3)}, 0x60, {VA(0)}"]


def set_ka_ins(sbase):
    return [f"v_add_u32 {KA(0)}, {sbase}, {KL0}", f"v_xor_b32 {KA(1)}, 32, {KA(0)}",
            f"v_xor_b32 {KA(2)}, 64, {KA(0)}", f"v_xor_b32 {KA(3)}, 0x60, {KA(0)}"]


def kread(kk):
    return f"ds_read_b128 {KR(kk % 4)}, {KA(kk & 3)} offset:{128 * (kk >> 2)}"


def plan_groups(nv_dst):
    """Scalar plan of the next tile to stream (its window lane is in S_LI):
    source base in S_B, valid row count in nv_dst (0 when its page is not a
    page of the pool: the tile is then streamed from page 0 and masked), and
    the page cursor advanced by one tile.  The lane select of v_readlane was
    written by SALU at least one instruction earlier."""
    return [
        [f"v_readlane_b32 {S_T0}, {PWIN}, {S_LI}"],
        [f"s_sub_i32 {nv_dst}, %[end], {S_U0}", f"s_min_i32 {nv_dst}, {nv_dst}, {TOK}"],
        [f"s_cmp_lt_u32 {S_T0}, %[npg]", f"s_cselect_b32 {S_T0}, {S_T0}, 0", f"s_cselect_b32 {nv_dst}, {nv_dst}, 0"],
        [f"s_mul_i32 {S_T0}, {S_T0}, %[P]", f"s_add_u32 {S_T0}, {S_T0}, {S_ON}"],
        [f"s_mul_i32 {S_T1}, {S_T0}, {ROW}", f"s_mul_hi_u32 {S_T2}, {S_T0}, {ROW}"],
        [f"s_add_u32 {S_B0}, %[kv_lo], {S_T1}", f"s_addc_u32 {S_B1}, %[kv_hi], {S_T2}"],
        [f"s_add_u32 {S_U0}, {S_U0}, {TOK}", f"s_add_u32 {S_ON}, {S_ON}, {TOK}"],
        [f"s_cmp_ge_u32 {S_ON}, %[P]", f"s_cselect_b32 {S_T1}, %[P], 0", f"s_cselect_b32 {S_T2}, 1, 0"],
        [f"s_sub_u32 {S_ON}, {S_ON}, {S_T1}", f"s_add_u32 {S_PN}, {S_PN}, {S_T2}"],
        [f"s_sub_u32 {S_LI}, {S_PN}, {S_PBASE}"],
    ]


def dma_groups(m0_base_sgpr):
    """Nine direct loads of the planned tile; load PI of wave w fills LDS
    chunk w + 4 PI (M0 needs one wait state before the load).  Dense tiles
    are read once per call from a pool larger than the Infinity Cache, so
    the loads are nontemporal: they do not allocate there, and so neither
    evict other data nor pay for writing back dirty lines they would
    displace.  (Sparse tile loads allocate: a batch's gathered rows fit in
    that cache and are read again by the next call.)"""
    return [[f"s_add_u32 m0, {m0_base_sgpr}, {4096 * pi}", "s_nop 0",
             f"global_load_lds_dwordx4 {LO(pi)}, {S_B} nt"] for pi in range(LOADS)]


def sparse_plan_groups(nv_dst):
    """Sparse plan of the next tile to stream (its index in the segment is in
    S_LI): its row-valid mask in nv_dst and the LDS address of its window
    values in S_WINU; the tile cursor advances by one."""
    return [
        [f"v_readlane_b32 {nv_dst}, {PWIN}, {S_LI}"],
        [f"s_lshl_b32 {S_WINU}, {S_LI}, 7", f"s_add_u32 {S_WINU}, {S_WINU}, {S_WINB}"],
        [f"s_add_u32 {S_LI}, {S_LI}, 1"],
    ]


def sparse_ew_read(pi, tmp):
    """Window value of the tile row of load pi's piece (4 x row in the high
    half of LO(pi)) into tmp."""
    return [f"v_add_u32_sdwa {tmp}, {S_WINU}, {LO(pi)} dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
            "src1_sel:WORD_1",
            f"ds_read_b32 {tmp}, {tmp}"]


def sparse_dma(pi, tmp, m0_base_sgpr):
    """Load pi of the planned sparse tile: window value + piece offset (low
    half of LO(pi)) from the pool base; the add is M0's wait state."""
    return [f"s_add_u32 m0, {m0_base_sgpr}, {4096 * pi}",
            f"v_add_u32_sdwa {tmp}, {tmp}, {LO(pi)} dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
            "src1_sel:WORD_0",
            f"global_load_lds_dwordx4 {tmp}, {S_B}"]


def window_load(em):
    """Block-table window: lane i holds the entry of page S_PBASE + i, or -1
    for pages at or past the segment's end (those are never loaded)."""
    em.op("v_mbcnt_lo_u32_b32 v208, -1, 0")
    em.op("v_mbcnt_hi_u32_b32 v208, -1, v208")
    em.op(f"v_add_u32 v208, {S_PBASE}, v208")
    em.op(f"v_mov_b32 {PWIN}, -1")
    em.op("v_cmp_gt_u32 vcc, %[pend], v208")
    em.op(f"s_and_saveexec_b64 {S_EXEC}, vcc")
    em.op("v_lshlrev_b32 v208, 2, v208")
    em.op(f"global_load_dword {PWIN}, v208, %[bt]")
    em.op(f"s_mov_b64 exec, {S_EXEC}")


def zero_masked_rows(em, nv_sgpr, buf_sgpr, tag, sparse=False):
    """Rows >= nv of the tile in the LDS buffer at buf_sgpr become zero
    (sparse: rows whose bit in the mask nv is clear).  Each wave clears the
    16-byte pieces its own nine loads wrote, which have landed (so no load
    can overwrite the zeros); the caller's barrier makes them visible."""
    if sparse:
        em.op(f"s_cmp_eq_u32 {nv_sgpr}, -1")
        em.op(f"s_cbranch_scc1 {em.ref('zskip_' + tag)}")
    else:
        em.op(f"s_cmp_lt_u32 {nv_sgpr}, {TOK}")
        em.op(f"s_cbranch_scc0 {em.ref('zskip_' + tag)}")
    for r in (212, 213, 214, 215):
        em.op(f"v_mov_b32 v{r}, 0")
    em.op("v_mbcnt_lo_u32_b32 v208, -1, 0")
    em.op("v_mbcnt_hi_u32_b32 v208, -1, v208")          # lane
    em.op(f"s_lshl_b32 {S_T1}, %[w], 6")
    em.op(f"v_add_u32 v209, {S_T1}, v208")               # p0 = 64 w + lane
    em.op("v_lshlrev_b32 v210, 4, v208")
    em.op(f"v_add_u32 v210, {S_LDSW}, v210")             # lds + 1024 w + 16 lane
    em.op(f"s_sub_u32 {S_T1}, {buf_sgpr}, %[lds]")
    em.op(f"v_add_u32 v210, {S_T1}, v210")               # + the buffer's offset
    for pi in range(LOADS):
        em.op(f"v_add_u32 v211, {256 * pi}, v209")
        em.op(f"v_mul_u32_u24 v211, {DIV72_MUL}, v211")
        em.op(f"v_lshrrev_b32 v211, {DIV72_SHIFT}, v211")   # row of this lane's piece
        if sparse:
            em.op(f"v_lshrrev_b32_e64 v211, v211, {nv_sgpr}")
            em.op("v_and_b32 v211, 1, v211")
            em.op("v_cmp_eq_u32 vcc, 0, v211")
        else:
            em.op(f"v_cmp_le_u32 vcc, {nv_sgpr}, v211")
        em.op(f"s_and_saveexec_b64 {S_EXEC}, vcc")
        em.lds(f"ds_write_b128 v210, v[212:215] offset:{4096 * pi}")
        em.op(f"s_mov_b64 exec, {S_EXEC}")
    em.wait_all()
    em.label("zskip_" + tag)


def mask_scores(em, p, nv_sgpr, tag, sparse=False):
    """Scores of rows >= nv (sparse: of rows whose mask bit is clear) become
    -inf (lane (n, hh) holds tokens 8 (e >> 2) + 4 hh + (e & 3) of head n);
    entered at least 16 wait states after the last MFMA that wrote the
    block."""
    if sparse:
        em.op(f"s_cmp_eq_u32 {nv_sgpr}, -1")
        em.op(f"s_cbranch_scc1 {em.ref('mskip_' + tag)}")
    else:
        em.op(f"s_cmp_lt_u32 {nv_sgpr}, {TOK}")
        em.op(f"s_cbranch_scc0 {em.ref('mskip_' + tag)}")
    em.op("s_nop 7")
    em.op("s_nop 7")
    em.op(f"v_mbcnt_lo_u32_b32 {T0}, -1, 0")
    em.op(f"v_mbcnt_hi_u32_b32 {T0}, -1, {T0}")
    em.op(f"v_lshrrev_b32 {T0}, 5, {T0}")
    em.op(f"v_lshlrev_b32 {T0}, 2, {T0}")                 # 4 hh
    if sparse:
        em.op(f"v_lshrrev_b32_e64 {T0}, {T0}, {nv_sgpr}")  # the lane's half of the mask
    em.op(f"v_mov_b32 {CV}, {NEG_INF}")
    for e in range(16):
        c = 8 * (e >> 2) + (e & 3)
        if sparse:
            em.op(f"v_bfe_u32 {T1}, {T0}, {c}, 1")
            em.op(f"v_cmp_ne_u32 vcc, 0, {T1}")
        else:
            em.op(f"v_add_u32 {T1}, {c}, {T0}")
            em.op(f"v_cmp_gt_u32 vcc, {nv_sgpr}, {T1}")
        em.op(f"v_cndmask_b32 {Se(p, e)}, {CV}, {Se(p, e)}, vcc")
    em.label("mskip_" + tag)


def mx_move_items(p, first, earliest):
    """Row max of score block p over the lane pair (of the raw scores: the
    scale is positive, so it is the max of the scaled scores), then the lazy
    reference move: m_ref, m_sub = m_ref - 7 (floored), alpha (1 when nothing
    moved) to LDS and kept in T0.  With `first` the accumulator is still zero
    and alpha is 1."""
    its = []
    prev = Item([f"v_max3_f32 {T0}, {Se(p, 0)}, {Se(p, 1)}, {Se(p, 2)}"], earliest)
    its.append(prev)
    for k in range(6):
        prev = Item([f"v_max3_f32 {T0}, {T0}, {Se(p, 3 + 2 * k)}, {Se(p, 4 + 2 * k)}"], deps=[(prev, 0)])
        its.append(prev)
    seq = [[f"v_max_f32 {T0}, {T0}, {Se(p, 15)}"],
           [f"v_mov_b32 {T1}, {T0}", "s_nop 1", f"v_permlane32_swap_b32 {T0}, {T1}"],
           [f"v_max_f32 {T0}, {T0}, {T1}"],
           [f"v_mul_f32 {T0}, %[scale], {T0}"],
           [f"v_add_f32 {T1}, {RESCALE_THR}, {M_REF}"],
           [f"v_cmp_gt_f32 vcc, {T0}, {T1}"],
           [f"v_sub_f32 {T1}, {M_REF}, {T0}", f"v_cndmask_b32 {T1}, 0, {T1}, vcc"],
           [f"v_exp_f32 {T1}, {T1}"],
           [f"v_cndmask_b32 {M_REF}, {M_REF}, {T0}, vcc"],
           [f"v_add_f32 {M_SUB}, {P_SHIFT_NEG}, {M_REF}"],
           [f"v_max_f32 {M_SUB}, {FLOOR}, {M_SUB}"]]
    if first:
        seq.append([f"v_mov_b32 {T1}, 1.0"])
    # alpha stays in T0 for the normaliser update l = l alpha + sum(p) in the
    # next step's S^T stream
    seq.append([f"v_mov_b32 {T0}, {T1}"])
    seq.append([f"ds_write_b32 {XW}, {T1}"])
    for g in seq:
        prev = Item(g, deps=[(prev, 0)])
        its.append(prev)
    return its


def vote_ins():
    """S_VOTE = lanes where one of the four alphas in v208..v211 is not 1.0.
    A float equals 1.0 exactly when its bits are 0x3f800000, so the test is
    on the bits: bitop3 0x7e is (src0 ^ src2) | (src1 ^ src2).  The alphas
    are consumed (the rescale reads them from LDS again); no scalar
    instruction waits on a vector compare."""
    return [f"v_bitop3_b32 v208, v208, v209, 1.0 bitop3:0x7e", f"v_bitop3_b32 v210, v210, v211, 1.0 bitop3:0x7e",
            f"v_or_b32 v208, v208, v210", f"v_cmp_ne_u32_e64 {S_VOTE}, 0, v208"]


def rescale(em):
    """acc tile T *= alpha of its head tile ((T & 3) + wave) & 3, per lane."""
    for g in range(4):
        em.op(f"s_add_u32 {S_T0}, %[w], {g}")
        em.op(f"s_and_b32 {S_T0}, {S_T0}, 3")
        em.op(f"s_lshl_b32 {S_T0}, {S_T0}, 2")
        em.op(f"v_add_u32 {CV}, {S_T0}, {XR}")
        em.lds(f"ds_read_b32 v{212 + g}, {CV}")
    em.wait_all()
    for t in range(16):
        g = t & 3
        for i0 in range(0, 16, 4):
            for i in range(4):
                em.op(f"v_accvgpr_read_b32 v{208 + i}, a{16 * t + i0 + i}")
            for i in range(4):
                em.op(f"v_mul_f32 v{208 + i}, v{208 + i}, v{212 + g}")
            for i in range(4):
                em.op(f"v_accvgpr_write_b32 a{16 * t + i0 + i}, v{208 + i}")
    em.op("s_nop 4")


# ---------------------------------------------------------------- one step


ST_LOADS = 4   # sparse: loads 0..3 of tile it+3 go in the S^T stream (address temporaries v212..v215)


def sparse_load_items(pis, temps, first_dep, earliest, read_dist):
    """Window reads and loads pi of `pis` (address temporary temps[k]) as
    placement items: the reads chained from first_dep, each load at least
    read_dist steps after its read and one step after the previous load."""
    reads, loads = [], []
    prev = first_dep
    for pi, tmp in zip(pis, temps):
        r = Item(sparse_ew_read(pi, tmp), earliest=earliest, deps=[(prev, 0)] if prev else [])
        reads.append(r)
        prev = r
    prev = first_dep
    for r, (pi, tmp) in zip(reads, zip(pis, temps)):
        deps = [(r, read_dist)] + ([(prev, 1 if prev in loads else 0)] if prev else [])
        ld = Item(sparse_dma(pi, tmp, S_M0B), earliest=earliest, deps=deps, wait=(lambda ri=r: ri.lds_idx))
        loads.append(ld)
        prev = ld
    return reads + loads


def step(em, name, cur, has_next, has_n2, has_n3, sparse=False):
    """Tile step `it`: S^T of tile it+1 (if any) with the softmax of tile it,
    then PV of tile it.  Entering: score block `cur` holds tile it's raw
    scores, m_sub/m_ref/l_run are moved for tile it, its alphas are in LDS,
    V^T (dt, 0) of tile it is in v176.. (fragments 0 and 1 converted),
    and its V^T addresses are in VA."""
    nxt = cur ^ 1
    em.comment(f"==== step {name}")
    em.label(name)
    if has_next:
        # K read addresses of tile it+1 (no data involved) ahead of the barrier
        for x in [f"s_add_u32 {S_KB}, {S_IT}, 1", f"s_and_b32 {S_KB}, {S_KB}, 3",
                  f"s_mul_i32 {S_KB}, {S_KB}, {TILE}", f"s_add_u32 {S_KB}, {S_KB}, %[lds]"]:
            em.op(x)
        for x in set_ka_ins(S_KB):
            em.op(x)
    em.op("s_waitcnt vmcnt(9)" if has_n2 else "s_waitcnt vmcnt(0)")
    em.op("s_waitcnt lgkmcnt(0)")
    em.reset()
    em.op("s_barrier")
    if has_next:
        kidx = {kk: em.lds(kread(kk)) for kk in range(KDEPTH)}
    if has_n3 and not sparse:
        em.op(f"s_cmp_lt_u32 {S_LI}, 64")
        em.op(f"s_cbranch_scc1 {em.ref('win_ok_' + name)}")
        em.op(f"s_mov_b32 {S_PBASE}, {S_PN}")
        window_load(em)
        em.op("s_waitcnt vmcnt(0)")
        em.op(f"s_mov_b32 {S_LI}, 0")
        em.label("win_ok_" + name)
    vote_idx = em.lds(f"ds_read_b128 {PR(0)}, {XR}")

    # -- hook groups of the S^T stream, in priority order
    items = []
    exps = []
    for e in range(16):
        it = Item([f"v_fma_f32 {Se(cur, e)}, {Se(cur, e)}, %[scale], -{M_SUB}",
                   f"v_exp_f32 {Se(cur, e)}, {Se(cur, e)}"], earliest=(e * 3) // 2)
        exps.append(it)
        items.append(it)
    if has_n3:
        # scalar plan and loads of tile it+3 (its buffer was freed at the top)
        prev = None
        for g in (sparse_plan_groups if sparse else plan_groups)(S_NV3):
            prev = Item(g, earliest=0, deps=[(prev, 0)] if prev else [])
            items.append(prev)
        prev = Item([f"s_add_u32 {S_T3}, {S_IT}, 3", f"s_and_b32 {S_T3}, {S_T3}, 3",
                     f"s_mul_i32 {S_T3}, {S_T3}, {TILE}", f"s_add_u32 {S_M0B}, {S_T3}, {S_LDSW}"],
                    deps=[(prev, 0)])
        items.append(prev)
        if sparse:
            # the first ST_LOADS loads here, the rest in the PV stream
            items += sparse_load_items(range(ST_LOADS), [f"v{212 + k}" for k in range(ST_LOADS)], prev, 0, 4)
    adds, cvts = [], []
    prev = None
    for e in range(1, 16):
        if e == 1:
            ins = [f"v_add_f32 {T1}, {Se(cur, 0)}, {Se(cur, 1)}"]
            deps = [(exps[0], 2), (exps[1], 2)]
        else:
            ins = [f"v_add_f32 {T1}, {T1}, {Se(cur, e)}"]
            deps = [(exps[e], 2), (prev, 0)]
        prev = Item(ins, deps=deps)
        adds.append(prev)
        items.append(prev)
        if e % 2 == 1:
            q = e // 2
            c = Item([f"v_cvt_pk_f16_f32 v{216 + q}, {Se(cur, 2 * q)}, {Se(cur, 2 * q + 1)}"],
                     deps=[(exps[2 * q], 2), (exps[2 * q + 1], 2)])
            cvts.append(c)
            items.append(c)
    lrun = Item([f"v_fma_f32 {L_RUN}, {L_RUN}, {T0}, {T1}"], deps=[(adds[-1], 0)])
    items.append(lrun)
    # the two P writes in shadows of their own (each costs an MFMA's shadow)
    pwrite0 = Item([f"ds_write_b128 {PW}, {PH(0)}"], deps=[(c, 1) for c in cvts[:4]])
    pwrite1 = Item([f"ds_write_b128 {PW}, {PH(1)} offset:1024"], deps=[(c, 1) for c in cvts[4:]])
    items += [pwrite0, pwrite1]
    items.append(Item(vote_ins(), earliest=12, wait=vote_idx))
    # V^T (2, 0) and (3, 0) of tile it to fp16 (read in the previous step)
    for dt in (2, 3):
        for g in conv_groups(V0_BASE + 4 * dt):
            items.append(Item(g, earliest=0))

    if has_next:
        slots = place(items, KSTEPS, HOOK_CAP_QK)
        v1_idx = []
        for kk in range(KSTEPS):
            em.wait(kidx[kk])
            src_c = "0" if kk == 0 else S(nxt)
            em.op(f"v_mfma_f32_32x32x16_bf16 {S(nxt)}, {KR(kk % 4)}, {Q(kk)}, {src_c}")
            if kk + KDEPTH < KSTEPS:
                kidx[kk + KDEPTH] = em.lds(kread(kk + KDEPTH))
            emit_items(em, slots[kk])
            if kk >= KSTEPS - 4:
                # V^T (dt, 1) of tile it into the K operand slot this MFMA
                # has just read (KR(dt) is V1(dt)); the reads stay in flight
                # across the barrier and land before the PV stream needs them
                dt = kk - (KSTEPS - 4)
                idx = None
                for x in vfrag_read_ins(V1_BASE + 4 * dt, dt, 1):
                    idx = em.lds(x)
                v1_idx.append(idx)
        # masked rows of tile it+1 (landed at the top) are cleared before any
        # wave reads its V^T (after the barrier).  That branch drains every
        # LDS operation; without it only the V^T reads above are in flight
        # (every older operation completed before the last MFMA's wait), so
        # the count is carried on as if the clearing did not happen.
        mark = (em.issued, em.done)
        zero_masked_rows(em, S_NV1, S_KB, name, sparse)
        em.issued, em.done = mark
    else:
        # last tile: the softmax alone; exps, then dependent work
        slots = place(items, KSTEPS, 64)
        for kk in range(KSTEPS):
            if slots[kk]:
                emit_items(em, slots[kk])
                em.op("s_nop 0")
    if has_next:
        # every LDS operation older than the V^T reads (the P writes among
        # them) is complete before the barrier
        em.wait(v1_idx[0] - 2)
    else:
        em.wait_all()
        em.reset()
        v1_idx = None
    em.op("s_barrier")
    em.op(f"s_cmp_lg_u64 {S_VOTE}, 0")
    em.op(f"s_cbranch_scc0 {em.ref('norescale_' + name)}")
    # the rescale drains every LDS operation; the count without it is kept
    mark = (em.issued, em.done)
    rescale(em)
    em.issued, em.done = mark
    em.label("norescale_" + name)
    pv(em, name, cur, nxt, has_next, has_n3, sparse, v1_idx)
    em.op(f"s_add_u32 {S_IT}, {S_IT}, 1")
    em.op(f"s_mov_b32 {S_NV1}, {S_NV2}")
    em.op(f"s_mov_b32 {S_NV2}, {S_NV3}")


def pv(em, name, cur, nxt, has_next, has_n3, sparse=False, v1_pre=None):
    """O^T += V^T P^T for tile it: MFMA q has j = q >> 4, group g =
    (q >> 2) & 3 (head tile (g + wave) & 3) and dim tile dt = q & 3.  Group 0
    takes this wave's own P from registers, groups 1..3 read theirs from LDS
    into two alternating slots."""
    preads = [(0, 1), (0, 2), (0, 3), (1, 1), (1, 2), (1, 3)]
    # four P slots: the two fragment slots and the upper half of the score
    # block of tile it (dead once the S^T stream has taken its P)
    pslots = [PR(0), PR(1), f"v[{S_BASE[cur] + 8}:{S_BASE[cur] + 11}]", f"v[{S_BASE[cur] + 12}:{S_BASE[cur] + 15}]"]
    slot_of = {jg: k % 4 for k, jg in enumerate(preads)}
    read_before = {8: 4, 12: 5}   # read k issued before MFMA q (its slot's last reader has issued)
    pidx = {}

    def pread(k):
        j, g = preads[k]
        pidx[(j, g)] = em.lds(f"ds_read_b128 {pslots[k % 4]}, {PRG(g)} offset:{1024 * j}")

    for k in range(4):
        pread(k)
    # V^T (dt, 1) of tile it (read in the S^T stream when there was one)
    if v1_pre is not None:
        v1_idx = list(v1_pre)
    else:
        v1_idx = []
        for dt in range(4):
            idx = None
            for x in vfrag_read_ins(V1_BASE + 4 * dt, dt, 1):
                idx = em.lds(x)
            v1_idx.append(idx)
    if has_next:
        mask_scores(em, nxt, S_NV1, name, sparse)

    items = []
    # V^T (dt, 1) conversions: fragment dt is first read by MFMA 16 + dt, and
    # a vector-ALU write needs two wait states before an MFMA reads it
    v1c = []
    for dt in range(4):
        for g in conv_groups(V1_BASE + 4 * dt):
            it = Item(g, earliest=0, wait=v1_idx[dt])
            it.frag = dt
            v1c.append(it)
            items.append(it)
    if has_n3 and sparse:
        # loads ST_LOADS.. of tile it+3; the address temporaries are the
        # current score block, dead once the S^T stream has taken its P
        pis = range(ST_LOADS, LOADS)
        items += sparse_load_items(pis, [Se(cur, k) for k in range(len(pis))], None, 1, 3)
    elif has_n3:
        # the nine loads of tile it+3 (planned in the S^T stream; its buffer
        # was freed at the top of the step)
        prev = None
        for g in dma_groups(S_M0B):
            prev = Item(g, earliest=1, deps=[(prev, 1)] if prev else [])
            items.append(prev)
    v0r = []
    if has_next:
        # V^T (dt, 0) of tile it+1: addresses (its LDS base is S_KB), reads once
        # phase 0 has issued (MFMA 15 is the last to read v176..v191); placed
        # ahead of the max chain so that they go out early
        setva = Item(set_va_ins(S_KB), earliest=15)
        items.append(setva)
        for dt in range(4):
            ins = vfrag_read_ins(V0_BASE + 4 * dt, dt, 0)
            it = Item(ins, earliest=16, deps=[(setva, 0)])
            v0r.append(it)
            items.append(it)
        items += mx_move_items(nxt, False, earliest=10)
        # V^T (0, 0) and (1, 0) of tile it+1 to fp16 here; (2, 0), (3, 0) in
        # the next step's S^T stream
        for dt in (0, 1):
            for g in conv_groups(V0_BASE + 4 * dt):
                items.append(Item(g, deps=[(v0r[dt], 3)], wait=(lambda ri=v0r[dt]: ri.lds_idx)))
    slots = place(items, 32, HOOK_CAP_PV)
    for it in v1c:
        assert it.step <= 14 + it.frag, "V^T (dt, 1) converted too late"
    for q in range(32):
        if q in read_before:
            pread(read_before[q])
        j, g, dt = q >> 4, (q >> 2) & 3, q & 3
        if g >= 1 and dt == 0:
            em.wait(pidx[(j, g)])
        a_op = V0(dt) if j == 0 else V1(dt)
        b_op = PH(j) if g == 0 else pslots[slot_of[(j, g)]]
        t = 4 * dt + g
        em.op(f"v_mfma_f32_32x32x16_f16 a[{16 * t}:{16 * t + 15}], {a_op}, {b_op}, a[{16 * t}:{16 * t + 15}]")
        for it in slots[q]:
            if it in v0r:
                assert q >= 16
            emit_items(em, [it])


# ---------------------------------------------------------------- segment


def prologue(em, sparse=False):
    em.op(f"s_mov_b32 {S_M0SAVE}, m0")
    em.op("v_mbcnt_lo_u32_b32 v208, -1, 0")
    em.op("v_mbcnt_hi_u32_b32 v208, -1, v208")      # lane
    em.op("v_and_b32 v209, 31, v208")               # n32
    em.op("v_lshrrev_b32 v210, 5, v208")            # hh
    # query offset: 1152 n32 + 16 hh
    em.op(f"v_mul_u32_u24 v211, {ROW}, v209")
    em.op("v_lshl_add_u32 v211, v210, 4, v211")
    # key(n32) = 4 ((n32 >> 1) & 1) + ((n32 >> 2) & 3)
    em.op("v_bfe_u32 v212, v209, 1, 1")
    em.op("v_bfe_u32 v213, v209, 2, 2")
    em.op("v_lshl_or_b32 v212, v212, 2, v213")
    # K lane offset: 1152 n32 + 16 (hh ^ key)
    em.op("v_xor_b32 v213, v210, v212")
    em.op(f"v_mul_u32_u24 {KL0}, {ROW}, v209")
    em.op(f"v_lshl_add_u32 {KL0}, v213, 4, {KL0}")
    # V^T lane offset (i16 = lane & 15, gp = (lane >> 4) & 1, hp = (i16 >> 1) & 1):
    # 1152 (4 hh + (i16 >> 2)) + 64 (i16 >> 3) + 32 gp + 16 (hp ^ hh) + 8 (i16 & 1) + 256 w
    em.op("v_and_b32 v212, 15, v208")
    em.op("v_bfe_u32 v213, v208, 4, 1")
    em.op("v_lshrrev_b32 v214, 2, v212")
    em.op("v_lshl_add_u32 v214, v210, 2, v214")
    em.op(f"v_mul_u32_u24 {VL0}, {ROW}, v214")
    em.op("v_lshrrev_b32 v214, 3, v212")
    em.op(f"v_lshl_add_u32 {VL0}, v214, 6, {VL0}")
    em.op(f"v_lshl_add_u32 {VL0}, v213, 5, {VL0}")
    em.op("v_bfe_u32 v214, v212, 1, 1")
    em.op("v_xor_b32 v214, v214, v210")
    em.op(f"v_lshl_add_u32 {VL0}, v214, 4, {VL0}")
    em.op("v_and_b32 v214, 1, v212")
    em.op(f"v_lshl_add_u32 {VL0}, v214, 3, {VL0}")
    em.op(f"s_lshl_b32 {S_T1}, %[w], 8")
    em.op(f"v_add_u32 {VL0}, {S_T1}, {VL0}")
    # P slots: pl + 2048 ht + 16 lane (write: ht = w; read group g: ht = (g + w) & 3)
    em.op("v_lshlrev_b32 v214, 4, v208")
    em.op(f"s_add_u32 {S_T1}, %[lds], {P_OFF}")
    em.op(f"v_add_u32 v214, {S_T1}, v214")
    em.op(f"s_lshl_b32 {S_T2}, %[w], 11")
    em.op(f"v_add_u32 {PW}, {S_T2}, v214")
    for g in (1, 2, 3):
        em.op(f"s_add_u32 {S_T2}, %[w], {g}")
        em.op(f"s_and_b32 {S_T2}, {S_T2}, 3")
        em.op(f"s_lshl_b32 {S_T2}, {S_T2}, 11")
        em.op(f"v_add_u32 {PRG(g)}, {S_T2}, v214")
    # alpha slots x[n32][ht]: read x + 16 n32, write + 4 w
    em.op(f"s_add_u32 {S_T1}, %[lds], {X_OFF}")
    em.op("v_lshlrev_b32 v214, 4, v209")
    em.op(f"v_add_u32 {XR}, {S_T1}, v214")
    em.op(f"s_lshl_b32 {S_T2}, %[w], 2")
    em.op(f"v_add_u32 {XW}, {S_T2}, {XR}")
    # load source offsets 16 (p ^ key(p / 72)), p = 64 w + lane + 256 PI
    em.op(f"s_lshl_b32 {S_T1}, %[w], 6")
    em.op(f"v_add_u32 v213, {S_T1}, v208")
    for pi in range(LOADS):
        em.op(f"v_add_u32 v214, {256 * pi}, v213")
        em.op(f"v_mul_u32_u24 v215, {DIV72_MUL}, v214")
        em.op(f"v_lshrrev_b32 v215, {DIV72_SHIFT}, v215")
        em.op("v_bfe_u32 v216, v215, 1, 1")
        em.op("v_bfe_u32 v217, v215, 2, 2")
        em.op("v_lshl_or_b32 v216, v216, 2, v217")
        em.op("v_xor_b32 v214, v214, v216")
        em.op(f"v_lshlrev_b32 {LO(pi)}, 4, v214")
        if sparse:
            em.op(f"v_lshl_or_b32 {LO(pi)}, v215, 18, {LO(pi)}")   # 4 x tile row in the high half
    em.op(f"s_lshl_b32 {S_T1}, %[w], 10")
    em.op(f"s_add_u32 {S_LDSW}, %[lds], {S_T1}")
    # segment state
    em.op(f"s_mov_b32 {S_IT}, 0")
    if sparse:
        em.op(f"s_mov_b32 {S_LI}, 0")
        em.op(f"s_add_u32 {S_WINB}, %[lds], {WIN_OFF}")
        em.op(f"s_mov_b32 {S_B0}, %[kv_lo]")
        em.op(f"s_mov_b32 {S_B1}, %[kv_hi]")
        for s in (S_NV1, S_NV2, S_NV3):
            em.op(f"s_mov_b32 {s}, -1")
        # tile masks: lane t (and t + 32) reads the mask of tile t
        em.op("v_and_b32 v214, 31, v208")
        em.op(f"s_add_u32 {S_T1}, %[lds], {MASK_OFF}")
        em.op(f"v_lshl_add_u32 v214, v214, 2, {S_T1}")
        em.lds(f"ds_read_b32 {PWIN}, v214")
    else:
        em.op(f"s_mov_b32 {S_PBASE}, %[pbase]")
        em.op(f"s_mov_b32 {S_PN}, %[pbase]")
        em.op(f"s_mov_b32 {S_ON}, %[on0]")
        em.op(f"s_mov_b32 {S_U0}, %[begin]")
        em.op(f"s_mov_b32 {S_LI}, 0")
        for s in (S_NV1, S_NV2, S_NV3):
            em.op(f"s_mov_b32 {s}, {TOK}")
        # window first, then the query (36 loads)
        window_load(em)
    for kk in range(KSTEPS):
        em.op(f"global_load_dwordx4 {Q(kk)}, v211, %[q] offset:{32 * kk}")
    for a in range(256):
        em.op(f"v_accvgpr_write_b32 a{a}, 0")
    em.op(f"v_mov_b32 {M_REF}, {NEG_INF}")
    em.op(f"v_mov_b32 {L_RUN}, 0")
    if sparse:
        em.wait_all()                                  # the masks have landed
    else:
        em.op(f"s_waitcnt vmcnt({KSTEPS})")          # the window has landed
    nv = [S_NV0, S_NV1, S_NV2]
    for t in range(3):
        if t > 0:
            em.op(f"s_cmp_gt_u32 %[ntiles], {t}")
            em.op(f"s_cbranch_scc0 {em.ref('pro_done')}")
        for g in (sparse_plan_groups if sparse else plan_groups)(nv[t]):
            for x in g:
                em.op(x)
        em.op(f"s_add_u32 {S_M0B}, {S_LDSW}, {t * TILE}")
        if sparse:
            # the nine window reads first (score blocks as temporaries), then the loads
            for pi in range(LOADS):
                for x in sparse_ew_read(pi, f"v{S_BASE[0] + pi}"):
                    em.op(x)
            em.wait_all()
            for pi in range(LOADS):
                for x in sparse_dma(pi, f"v{S_BASE[0] + pi}", S_M0B):
                    em.op(x)
        else:
            for g in dma_groups(S_M0B):
                for x in g:
                    em.op(x)
    em.label("pro_done")
    em.reset()
    # the query and tile 0 have landed once only the loads of tiles 1, 2 are younger
    em.op("s_cmp_ge_u32 %[ntiles], 3")
    em.op(f"s_cbranch_scc0 {em.ref('pro_w2')}")
    em.op("s_waitcnt vmcnt(18)")
    em.op(f"s_branch {em.ref('pro_w')}")
    em.label("pro_w2")
    em.op("s_cmp_eq_u32 %[ntiles], 2")
    em.op(f"s_cbranch_scc0 {em.ref('pro_w1')}")
    em.op("s_waitcnt vmcnt(9)")
    em.op(f"s_branch {em.ref('pro_w')}")
    em.label("pro_w1")
    em.op("s_waitcnt vmcnt(0)")
    em.label("pro_w")
    em.op("s_barrier")
    em.op(f"s_mov_b32 {S_KB}, %[lds]")
    zero_masked_rows(em, S_NV0, S_KB, "pro", sparse)
    # S^T of tile 0 into score block 0
    for x in set_ka_ins(S_KB):
        em.op(x)
    kidx = {kk: em.lds(kread(kk)) for kk in range(KDEPTH)}
    for kk in range(KSTEPS):
        em.wait(kidx[kk])
        src_c = "0" if kk == 0 else S(0)
        em.op(f"v_mfma_f32_32x32x16_bf16 {S(0)}, {KR(kk % 4)}, {Q(kk)}, {src_c}")
        if kk + KDEPTH < KSTEPS:
            kidx[kk + KDEPTH] = em.lds(kread(kk + KDEPTH))
    em.wait_all()
    em.op("s_barrier")                                # masked rows of tile 0 are cleared
    em.reset()
    for x in set_va_ins(S_KB):
        em.op(x)
    v0i = []
    for dt in range(4):
        idx = None
        for x in vfrag_read_ins(V0_BASE + 4 * dt, dt, 0):
            idx = em.lds(x)
        v0i.append(idx)
    for dt in (0, 1):
        em.wait(v0i[dt])
        for g in conv_groups(V0_BASE + 4 * dt):
            for x in g:
                em.op(x)
    mask_scores(em, 0, S_NV0, "pro", sparse)
    em.op("s_nop 7")
    em.op("s_nop 7")
    for it in mx_move_items(0, True, 0):
        for x in it.ins:
            em.op(x)
    em.wait_all()
    em.reset()
    em.op(f"s_mov_b32 {S_VOTE_LO}, 0")
    em.op(f"s_mov_b32 {S_VOTE_HI}, 0")


def generate(sparse=False):
    em = Emitter()
    em.comment("segment prologue (sparse)" if sparse else "segment prologue")
    prologue(em, sparse)
    em.op("s_cmp_ge_u32 %[ntiles], 4")
    em.op(f"s_cbranch_scc1 {em.ref('MA')}")
    em.op("s_cmp_eq_u32 %[ntiles], 3")
    em.op(f"s_cbranch_scc1 {em.ref('T3')}")
    em.op("s_cmp_eq_u32 %[ntiles], 2")
    em.op(f"s_cbranch_scc0 {em.ref('T1')}")
    for e in range(0, 16, 2):
        em.op(f"v_mov_b64 v[{S_BASE[1] + e}:{S_BASE[1] + e + 1}], v[{S_BASE[0] + e}:{S_BASE[0] + e + 1}]")
    em.op(f"s_branch {em.ref('T2')}")
    # steady state: two bodies with the score blocks swapped
    step(em, "MA", 0, True, True, True, sparse)
    em.op(f"s_add_u32 {S_T0}, {S_IT}, 3")
    em.op(f"s_cmp_lt_u32 {S_T0}, %[ntiles]")
    em.op(f"s_cbranch_scc1 {em.ref('MB')}")
    for e in range(0, 16, 2):
        em.op(f"v_mov_b64 v[{S_BASE[0] + e}:{S_BASE[0] + e + 1}], v[{S_BASE[1] + e}:{S_BASE[1] + e + 1}]")
    em.op(f"s_branch {em.ref('T3')}")
    step(em, "MB", 1, True, True, True, sparse)
    em.op(f"s_add_u32 {S_T0}, {S_IT}, 3")
    em.op(f"s_cmp_lt_u32 {S_T0}, %[ntiles]")
    em.op(f"s_cbranch_scc1 {em.ref('MA')}")
    # the last three tiles (no further loads)
    step(em, "T3", 0, True, True, False, sparse)
    step(em, "T2", 1, True, False, False, sparse)
    step(em, "T1", 0, False, False, False, sparse)
    em.op("s_waitcnt lgkmcnt(0)")
    em.op(f"s_mov_b32 m0, {S_M0SAVE}")
    return "\n".join(em.lines) + "\n"


def clobber_list():
    v = [f'"v{i}"' for i in range(256) if i not in (224, 225)]
    a = [f'"a{i}"' for i in range(256)]
    s = [f'"{x}"' for x in OWNED_SGPRS]
    # EXEC leaves the block as it entered (masked sections restore it) and M0
    # is saved and restored, so neither is listed.
    return ", ".join(v + a + s + ['"vcc"', '"scc"', '"memory"'])


def asm_macro(name, body):
    esc = body.replace("\\", "\\\\").replace('"', '\\"')
    out = [f"#define {name} \\"]
    for l in esc.rstrip("\n").split("\n"):
        out.append(f'  "{l}\\n" \\')
    out.append('  ""')
    return out


def header_text():
    out = ["// Generated by gen_mla_h128.py (the build runs it); do not edit.", "#pragma once"]
    out += asm_macro("ISK_H128_SEG_ASM", generate())
    out += asm_macro("ISK_H128_SPARSE_SEG_ASM", generate(sparse=True))
    out.append("#define ISK_H128_SEG_CLOBBERS " + clobber_list())
    out.append(f"#define ISK_H128_LDS_BYTES {LDS_BYTES}")
    out.append(f"#define ISK_H128_SPARSE_LDS_BYTES {SPARSE_LDS_BYTES}")
    out.append(f"#define ISK_H128_WIN_OFF {WIN_OFF}")
    out.append(f"#define ISK_H128_MASK_OFF {MASK_OFF}")
    out.append(f"#define ISK_H128_WIN_SLOTS {WIN_SLOTS}")
    return "\n".join(out) + "\n"


def write_header(path):
    txt = header_text()
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    old = open(path).read() if os.path.exists(path) else None
    if old != txt:
        with open(path, "w") as f:
            f.write(txt)
    return path


if __name__ == "__main__":
    print(write_header(sys.argv[1] if len(sys.argv) > 1 else "mla_h128_seg.inc"))
