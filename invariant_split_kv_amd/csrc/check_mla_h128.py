"""Static checker of the generated segment body of the dense 128-head MLA
kernel (the text gen_mla_h128.generate() returns).

The body is hand-scheduled: the generator places every LDS read, wait,
conversion and load itself, so an ordering mistake compiles fine and only
shows as wrong numbers.  This checker walks the body the way one wave
executes it for a given segment length -- branches are followed with the
scalar registers emulated, the lazy-rescale branch by a chosen policy -- and
checks, instruction by instruction:

  * load-use: no instruction reads or overwrites a VGPR whose LDS or vector
    memory load is still outstanding under the waits issued so far (LDS
    operations and vector loads each complete in issue order);
  * MFMA latency: no VALU instruction reads an accumulator or VGPR written by
    an MFMA fewer than MFMA_WAIT wait states earlier;
  * operand provenance: each S^T MFMA reads K from the LDS buffer of the tile
    it scores and the query from its loads; each PV MFMA reads the V^T
    fragment (dt, j) its accumulator tile needs, from the current tile's
    buffer, converted from bf16 to fp16 exactly once;
  * tile buffers: no LDS read of a buffer before this wave's direct loads
    into it have landed and a barrier has passed, and no direct load into a
    buffer before a barrier has passed since this wave's last read of it;
  * tile loads: each direct load uses the source offset of the piece slot
    its LDS destination names; in the sparse body it adds that offset to
    the window value of its tile row, read for the tile whose buffer it
    fills (tile it+3 in the steps), and the row-valid mask tested before a
    tile's rows are cleared or its scores masked is that tile's.

Used by the build (a failing check stops it) and by the CPU tests.
"""

import re
import sys

import gen_mla_h128 as g

MFMA_WAIT = 12   # wait states from a 32x32x16 MFMA result to a VALU read of it
STEP_LABELS = ("MA", "MB", "T3", "T2", "T1")
NO_DST = ("ds_write", "s_cmp", "global_load_lds", "s_waitcnt", "s_barrier", "s_nop", "s_branch", "s_cbranch",
          "global_store")
_REG = re.compile(r"^(v|a|s)(\d+)$|^(v|a|s)\[(\d+):(\d+)\]$")
K_ADDR = ("v230", "v231", "v232", "v233")
V_ADDR = ("v235", "v236", "v237", "v238")


def _regs(tok):
    tok = tok.strip()
    m = _REG.match(tok)
    if not m:
        return [tok] if tok in ("vcc", "exec", "m0") else []
    if m.group(1):
        return [f"{m.group(1)}{m.group(2)}"]
    return [f"{m.group(3)}{i}" for i in range(int(m.group(4)), int(m.group(5)) + 1)]


def sparse_mask(t):
    """Row-valid mask the checker gives tile t of a sparse segment: mostly
    full, some partial, some empty, so that every branch is taken."""
    if t % 7 == 5:
        return 0
    if t % 3 == 1:
        return (0xFFFFFFFF >> (t % 5 + 1)) ^ (1 << (t % 4))
    return 0xFFFFFFFF


class _Wave:
    def __init__(self, lines, inputs, rescale, sparse=False):
        self.lines = lines
        self.inp = inputs
        self.rescale = rescale
        self.sparse = sparse
        self.mask_tile = {}     # SGPR -> tile whose row-valid mask it holds (sparse)
        self.sg = {}
        self.scc = None
        self.lgkm = []          # outstanding LDS ops: (dst regs, buffer read or None)
        self.vm = []            # outstanding vector loads: (dst regs, buffer written or None)
        self.tag = {}
        self.mfma_at = {}
        self.clock = 0
        self.in_steps = False
        self.buf_state = {}     # buffer -> "pending" | "landed" | "visible"
        self.read_unfenced = set()   # buffers read since the last barrier
        self.errors = []
        self.labels = {l[:-1]: i for i, l in enumerate(lines) if l.endswith(":")}

    # -- helpers
    def err(self, i, msg):
        self.errors.append(f"line {i}: {self.lines[i].strip()} -- {msg} (tile {self.sg.get(g.S_IT)})")

    def val(self, tok):
        tok = tok.strip()
        if tok.startswith("%["):
            return self.inp.get(tok[2:-1])
        if re.match(r"^-?\d+$", tok):
            return int(tok) & 0xFFFFFFFF
        if re.match(r"^0x[0-9a-fA-F]+$", tok):
            return int(tok, 16)
        if re.match(r"^s\d+$", tok) or tok == "m0":
            return self.sg.get(tok)
        return None

    def buffer_of(self, addr_value):
        if addr_value is None:
            return None
        return (addr_value - self.inp["lds"]) // g.TILE

    def retire(self, queue, n):
        while len(queue) > n:
            _, buf = queue.pop(0)
            if queue is self.vm and buf is not None and not any(b == buf for _, b in self.vm):
                self.buf_state[buf] = "landed"

    # -- execution
    def run(self, limit=3_000_000):
        pc, n = 0, 0
        while pc < len(self.lines):
            n += 1
            if n > limit:
                raise RuntimeError("the body did not finish")
            line = self.lines[pc].strip()
            if line.endswith(":") and line.split("_%=")[0] in STEP_LABELS:
                self.in_steps = True
            if not line or line.startswith(";") or line.endswith(":"):
                pc += 1
                continue
            nxt = self.step(pc, line)
            pc = pc + 1 if nxt is None else nxt
        if self.lgkm or any(True for _ in self.vm):
            self.errors.append("the body ends with loads outstanding")
        return self.errors

    def step(self, i, line):
        op, _, rest = line.partition(" ")
        ops = [x.strip() for x in rest.split(",")] if rest else []
        mods = []
        if ops:
            parts = ops[-1].split()
            ops[-1], mods = parts[0], parts[1:]
        if op == "s_nop":
            self.clock += int(ops[0]) + 1
            return None
        self.clock += 1
        if op == "s_waitcnt":
            for m in re.finditer(r"(lgkmcnt|vmcnt)\((\d+)\)", rest):
                self.retire(self.lgkm if m.group(1) == "lgkmcnt" else self.vm, int(m.group(2)))
            return None
        if op == "s_barrier":
            for b, st in list(self.buf_state.items()):
                if st == "landed":
                    self.buf_state[b] = "visible"
            pending_reads = {b for _, b in self.lgkm if b is not None}
            self.read_unfenced &= pending_reads
            return None
        if op == "s_branch":
            return self.labels[ops[0]]
        if op.startswith("s_cbranch_scc"):
            lab = ops[0]
            if lab.startswith("norescale_"):
                return None if self.rescale(self) else self.labels[lab]
            if self.scc is None:
                self.err(i, "branch on an unknown condition")
                return None
            return self.labels[lab] if self.scc == op.endswith("1") else None

        if op.startswith("v_permlane32_swap"):
            dst = src = _regs(ops[0]) + _regs(ops[1])
        elif op.startswith(NO_DST):
            dst, src = [], [r for o in ops for r in _regs(o)]
        else:
            dst = _regs(ops[0]) if ops else []
            src = [r for o in ops[1:] for r in _regs(o)]
        pending = set()
        for regs, _ in self.lgkm + self.vm:
            pending |= regs
        for r in src:
            if r in pending:
                self.err(i, f"reads {r} while its load is outstanding")
            if (r in self.mfma_at and not op.startswith("v_mfma")
                    and self.clock - self.mfma_at[r] < MFMA_WAIT):
                self.err(i, f"reads {r} {self.clock - self.mfma_at[r]} wait states after the MFMA writing it")
        for r in dst:
            if r in pending:
                self.err(i, f"overwrites {r} while a load into it is outstanding")

        if op.startswith("ds_"):
            return self.lds_op(i, op, ops, mods, dst)
        if op.startswith("global_load_lds"):
            buf = self.buffer_of(self.sg.get("m0"))
            if buf is None:
                self.err(i, "direct load with an unknown LDS destination")
            elif buf in self.read_unfenced:
                self.err(i, f"direct load into buffer {buf} with no barrier since this wave read it")
            self.check_load_source(i, ops[0], buf)
            self.buf_state[buf] = "pending"
            self.vm.append((set(), buf))
            return None
        if op.startswith("global_load"):
            self.vm.append((set(dst), None))
            for r in dst:
                self.tag[r] = ("global",)
            return None
        if op.startswith("v_mfma"):
            self.mfma(i, op, ops)
            return None
        if op.startswith("s_"):
            self.salu(i, op, ops)
            return None
        return self.valu(i, op, ops, dst)

    def expected_tile(self, ahead):
        it = self.sg.get(g.S_IT)
        return None if it is None else it + ahead

    def check_load_source(self, i, vaddr, buf):
        """The piece slot the LDS destination names, and the offset used."""
        m0 = self.sg.get("m0")
        if buf is None or m0 is None:
            return
        rel = m0 - self.inp["lds"] - g.TILE * buf - 1024 * self.inp["w"]
        if rel % 4096 != 0 or not 0 <= rel // 4096 < g.LOADS:
            self.err(i, f"LDS destination {m0} is not a piece row of this wave")
            return
        pi = rel // 4096
        if not self.sparse:
            if vaddr != g.LO(pi):
                self.err(i, f"load {pi} of a tile uses offset {vaddr}, not {g.LO(pi)}")
            return
        tg = self.tag.get(vaddr) or ("",)
        if tg[0] != "ld_addr" or tg[2] != pi:
            self.err(i, f"load {pi} of a tile uses {vaddr} holding {tg}")
            return
        tile = tg[1]
        want = self.expected_tile(3) if self.in_steps else buf
        if tile is None or tile & 3 != buf or tile != want:
            self.err(i, f"load into buffer {buf} reads the window of tile {tile} (expected {want})")

    def check_mask(self, i, sreg):
        """A row-valid mask is tested for the tile about to be cleared or scored."""
        want = self.expected_tile(1) if self.in_steps else 0
        have = self.mask_tile.get(sreg)
        if have != want:
            self.err(i, f"mask in {sreg} is tile {have}'s, expected tile {want}'s")

    def lds_op(self, i, op, ops, mods, dst):
        buf = None
        if op == "ds_read_b32" and self.sparse:
            tg = self.tag.get(ops[1]) or ("",)
            if tg[0] == "ew_addr":
                self.lgkm.append((set(dst), None))
                for r in dst:
                    self.tag[r] = ("ew",) + tg[1:]
                    self.mfma_at.pop(r, None)
                return None
        if op.startswith("ds_read"):
            addr = ops[1]
            if addr in K_ADDR or addr in V_ADDR:
                buf = self.buffer_of(self.tag.get(addr))
                st = self.buf_state.get(buf)
                if st is not None and st != "visible":
                    self.err(i, f"reads tile buffer {buf} whose direct loads are {st}")
                self.read_unfenced.add(buf)
            off = int(mods[0].split(":")[1]) if mods else 0
            if op.startswith("ds_read_b64_tr_b16"):
                j = off // (g.ROW * 16)
                dt = 2 * ((off % (g.ROW * 8)) // 128) + V_ADDR.index(addr) // 2
                for r in dst:
                    self.tag[r] = ("v_bf16", buf, j, dt)
            elif addr in K_ADDR:
                for r in dst:
                    self.tag[r] = ("k", buf)
            else:
                for r in dst:
                    self.tag[r] = ("lds",)
        self.lgkm.append((set(dst) if op.startswith("ds_read") else set(), buf))
        for r in dst:
            self.mfma_at.pop(r, None)
        return None

    def mfma(self, i, op, ops):
        acc, a_op, b_op = _regs(ops[0]), _regs(ops[1]), _regs(ops[2])
        it = self.sg.get(g.S_IT)
        if "bf16" in op:
            want = 0 if not self.in_steps else (None if it is None else (it + 1) & 3)
            if any(self.tag.get(r) != ("k", want) for r in a_op):
                self.err(i, f"K operand is {self.tag.get(a_op[0])}, expected tile buffer {want}")
            if any(self.tag.get(r) != ("global",) for r in b_op):
                self.err(i, f"query operand is {self.tag.get(b_op[0])}")
        else:
            tile = int(acc[0][1:]) // 16
            want = ("v_f16", None if it is None else it & 3, 0 if int(a_op[0][1:]) < g.V1_BASE else 1, tile >> 2)
            if any(self.tag.get(r) != want for r in a_op):
                self.err(i, f"V operand is {self.tag.get(a_op[0])}, expected {want}")
        for r in acc:
            self.mfma_at[r] = self.clock

    def valu(self, i, op, ops, dst):
        if op == "v_and_b32" and ops[1] == "0xffff0000":
            src = _regs(ops[2])[0]
            if (self.tag.get(src) or ("",))[0] != "v_bf16":
                self.err(i, f"bf16 conversion of {src}, which holds {self.tag.get(src)}")
            self.tag[dst[0]] = ("tmp",)
        elif op == "v_lshlrev_b32" and ops[1] == "16":
            src = _regs(ops[2])[0]
            tg = self.tag.get(src) or ("",)
            if tg[0] != "v_bf16":
                self.err(i, f"bf16 conversion of {src}, which holds {tg}")
            self.tag[dst[0]] = ("v_shifted",) + tuple(tg[1:])
        elif op == "v_cvt_pkrtz_f16_f32":
            src = _regs(ops[1])[0]
            tg = self.tag.get(src) or ("",)
            if tg[0] != "v_shifted":
                self.err(i, f"fp16 pack of {src}, which holds {tg}")
            self.tag[dst[0]] = ("v_f16",) + tuple(tg[1:])
        elif op == "v_add_u32" and dst and dst[0] in (K_ADDR[0], V_ADDR[0]):
            self.tag[dst[0]] = self.val(ops[1])
        elif op == "v_xor_b32" and dst and (dst[0] in K_ADDR[1:] or dst[0] in V_ADDR[1:]):
            self.tag[dst[0]] = self.tag.get(_regs(ops[2])[0])
        elif op == "v_readlane_b32":
            if self.sparse:
                t = self.sg.get(ops[2])
                self.sg[ops[0]] = None if t is None else sparse_mask(t)
                self.mask_tile[ops[0]] = t
            else:
                self.sg[ops[0]] = 0     # block-table entry: page 0, a page of the pool
        elif op == "v_add_u32_sdwa":
            line = self.lines[i]
            src0, src1 = _regs(ops[1]), _regs(ops[2])
            pi = g.LO_REGS.index(src1[0]) if src1 and src1[0] in g.LO_REGS else None
            if "src1_sel:WORD_1" in line and ops[1] == g.S_WINU:
                base = self.sg.get(g.S_WINU)
                winb = self.sg.get(g.S_WINB)
                tile = None if base is None or winb is None or (base - winb) % 128 else (base - winb) // 128
                self.tag[dst[0]] = ("ew_addr", tile, pi)
            elif "src1_sel:WORD_0" in line and src0:
                tg = self.tag.get(src0[0]) or ("",)
                if tg[0] != "ew" or tg[2] != pi:
                    self.err(i, f"piece offset {pi} added to {src0[0]} holding {tg}")
                    self.tag[dst[0]] = ("valu",)
                else:
                    self.tag[dst[0]] = ("ld_addr", tg[1], pi)
            else:
                self.err(i, "unexpected SDWA form")
        else:
            if op == "v_lshrrev_b32_e64" and self.sparse and re.match(r"^s\d+$", ops[2]):
                self.check_mask(i, ops[2])
            for r in dst:
                self.tag[r] = ("valu",)
        for r in dst:
            self.mfma_at.pop(r, None)
        return None

    def salu(self, i, op, ops):
        v = [self.val(o) for o in ops]
        d = ops[0] if ops else None

        def put(x):
            if d is not None and (re.match(r"^s\d+$", d) or d == "m0"):
                self.sg[d] = None if x is None else x & 0xFFFFFFFF
                if op != "s_mov_b32":
                    self.mask_tile.pop(d, None)   # no longer a tile's mask

        def two(f):
            return None if v[1] is None or v[2] is None else f(v[1], v[2])

        def signed(x):
            return x - (1 << 32) if x >= 1 << 31 else x

        if op == "s_mov_b32":
            put(v[1])
            if d in self.mask_tile or ops[1] in self.mask_tile:
                self.mask_tile[d] = self.mask_tile.get(ops[1])
        elif op in ("s_add_u32", "s_add_i32"):
            put(two(lambda a, b: a + b))
        elif op in ("s_sub_u32", "s_sub_i32"):
            put(two(lambda a, b: a - b))
        elif op == "s_and_b32":
            put(two(lambda a, b: a & b))
        elif op == "s_mul_i32":
            put(two(lambda a, b: a * b))
        elif op == "s_lshl_b32":
            put(two(lambda a, b: a << b))
        elif op == "s_min_i32":
            put(two(lambda a, b: min(signed(a), signed(b))))
        elif op == "s_cselect_b32":
            put(None if self.scc is None else (v[1] if self.scc else v[2]))
        elif op.startswith("s_cmp_"):
            a, b = v[0], v[1]
            if self.sparse and op == "s_cmp_eq_u32" and ops[1] == "-1":
                self.check_mask(i, ops[0])
            kind = op.split("_")[2]
            if a is None or b is None:
                self.scc = None
            else:
                self.scc = {"lt": a < b, "ge": a >= b, "gt": a > b, "le": a <= b, "eq": a == b, "lg": a != b}[kind]
        elif op in ("s_mov_b64", "s_and_saveexec_b64", "s_or_b64", "s_addc_u32", "s_mul_hi_u32"):
            pass
        else:
            self.err(i, f"instruction {op} is not modelled")


def check_segment(body, tokens, begin=0, page=64, rescale="never", wave=1, sparse=False):
    """Errors found when one wave runs `body` over a segment of `tokens`
    tokens starting at `begin` (rescale: "never", "always" or "alternate");
    a sparse body gets the tile masks of sparse_mask."""
    end = begin + tokens
    inputs = dict(ntiles=(tokens + g.TOK - 1) // g.TOK, begin=begin, end=end, P=page, npg=1 << 20,
                  pbase=begin // page, on0=begin % page, pend=(end + page - 1) // page, lds=0, w=wave,
                  kv_lo=0, kv_hi=0)
    count = [0]

    def policy(_):
        count[0] += 1
        return {"never": False, "always": True, "alternate": count[0] % 2 == 0}[rescale]

    return _Wave(body.split("\n"), inputs, policy, sparse).run()


# (tokens, first token, page size): fewer than 4 tiles, each tail step after
# the steady state, both steady-state bodies, ragged tails, a split that
# starts inside a page, and block-table window reloads (more than 64 pages).
SEGMENTS = [(n, 0, 64) for n in (1, 31, 32, 33, 64, 65, 96, 97, 128, 129, 160, 191, 192, 256, 511, 512, 513)] + \
    [(300, 1600, 128), (4200, 0, 64), (9000, 1536, 128)]


# sparse segments: slot counts up to the window's 1024
SPARSE_SEGMENTS = [(n, 0, 64) for n in (1, 31, 32, 33, 64, 65, 96, 97, 128, 129, 160, 191, 192, 256, 511, 512,
                                         513, 1000, 1024)]


def check(body=None, segments=SEGMENTS, sparse=False):
    """All errors over `segments` under the three rescale policies."""
    body = g.generate(sparse=sparse) if body is None else body
    errors = []
    for n, begin, page in segments:
        # long segments repeat the steady state; one policy covers them
        for pol in ("never", "always", "alternate") if n <= 600 else ("alternate",):
            for e in check_segment(body, n, begin=begin, page=page, rescale=pol, sparse=sparse):
                errors.append(f"[{'sparse ' if sparse else ''}{n} tokens from {begin}, page {page}, "
                              f"rescale {pol}] {e}")
    return errors


def check_all():
    """The dense body over SEGMENTS and the sparse body over SPARSE_SEGMENTS."""
    return check() + check(segments=SPARSE_SEGMENTS, sparse=True)


if __name__ == "__main__":
    errs = check_all()
    for e in errs[:40]:
        print(e)
    print(f"{len(errs)} errors")
    sys.exit(1 if errs else 0)
