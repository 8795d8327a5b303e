"""A lane-level emulator of gfx950 kernel assembly (hipcc -S output), for replaying the
library's kernels on the CPU.

It implements the instructions the attention kernels compile to: scalar and vector ALU
ops, compares and EXEC masking, branches, s_waitcnt, s_barrier, scalar loads, global and
scratch loads and stores, LDS reads and writes (ds_read_b64_tr_b16 included), the
LDS-DMA copy global_load_lds_dwordx4, v_mfma_f32_32x32x16 / 16x16x32 (bf16, fp16) and
the AccVGPR moves.  Waves of a work group run in turn up to each barrier.

Memory results are held back until an s_waitcnt retires them (vector memory and LDS /
scalar memory each complete in issue order), so the replay sees what the hardware
guarantees and nothing more.  It raises

  * ``Fault`` for a global, scratch or LDS access outside its allocation, and for an
    LDS-DMA copy at or above ``LDS_COPY_LIMIT``;
  * ``Hazard`` for a read or overwrite of a register whose load is still in flight, an
    LDS access to bytes an unfinished copy of the same wave is writing, and two waves
    touching the same LDS byte (at least one writing) between two barriers, where a
    copy counts as writing until the wait that retires it;

and it records as a note (``Machine.notes``) any lane mask made by a compare that is
later combined with an EXEC holding lanes the compare did not see.  A compare writes 0
for inactive lanes, so such a use reads "false" for lanes that were never evaluated:
code that branches on ``exec & mask`` can then take the wrong side.
"""
from __future__ import annotations

import re
import struct

import numpy as np

M32 = 0xFFFFFFFF
M64 = 0xFFFFFFFFFFFFFFFF
LANES = 64
U32, U64, I32 = np.uint32, np.uint64, np.int32
# Asynchronous LDS copies of the library target only the first 64 KB of a work group's LDS
# (the rule that followed a GPU fault of a build copying into 64-128 KB); a replayed copy
# above it is reported as a fault.
LDS_COPY_LIMIT = 64 * 1024
# Initial byte of every lane's private (scratch) memory.  A read of scratch bytes never
# written is noted; replaying with another fill shows whether such a read can matter.
PRIV_FILL = 0


class Fault(Exception):
    """An access outside its allocation."""


class Hazard(Exception):
    """A use of a value the hardware does not guarantee to be there yet."""


# ---------------------------------------------------------------- parsing
class Operand:
    __slots__ = ("kind", "idx", "n", "neg", "abs", "val")

    def __init__(self, kind, idx=0, n=1, neg=False, ab=False, val=None):
        self.kind, self.idx, self.n, self.neg, self.abs, self.val = kind, idx, n, neg, ab, val

    def __repr__(self):
        return f"{self.kind}{self.idx}:{self.n}" if self.kind in "sva" else f"{self.kind}({self.val})"


_FLOAT_CONST = {"0.5": 0.5, "-0.5": -0.5, "1.0": 1.0, "-1.0": -1.0, "2.0": 2.0, "-2.0": -2.0,
                "4.0": 4.0, "-4.0": -4.0, "0.15915494": 0.15915494}
_SPECIAL = ("vcc", "exec", "vcc_lo", "vcc_hi", "exec_lo", "exec_hi", "m0", "off", "scc", "null")


def parse_operand(tok: str) -> Operand:
    tok = tok.strip()
    neg = False
    if tok.startswith("-") and tok[1:2] in ("v", "s", "a", "|"):
        neg, tok = True, tok[1:]
    ab = False
    if tok.startswith("|") and tok.endswith("|"):
        ab, tok = True, tok[1:-1]
    m = re.match(r"^([sva])(\d+)$", tok)
    if m:
        return Operand(m.group(1), int(m.group(2)), 1, neg, ab)
    m = re.match(r"^([sva])\[(\d+):(\d+)\]$", tok)
    if m:
        a, b = int(m.group(2)), int(m.group(3))
        return Operand(m.group(1), a, b - a + 1, neg, ab)
    if tok in _SPECIAL:
        return Operand(tok, neg=neg, ab=ab)
    if tok in _FLOAT_CONST:
        return Operand("f", val=_FLOAT_CONST[tok], neg=neg, ab=ab)
    if re.match(r"^-?0x[0-9a-fA-F]+$", tok):
        return Operand("i", val=int(tok, 16), neg=neg, ab=ab)
    if re.match(r"^-?\d+$", tok):
        return Operand("i", val=int(tok), neg=neg, ab=ab)
    if re.match(r"^-?\d+\.\d*(e-?\d+)?$", tok):
        return Operand("f", val=float(tok), neg=neg, ab=ab)
    raise ValueError(f"operand {tok!r}")


class Instr:
    __slots__ = ("op", "args", "mods", "line", "text")

    def __init__(self, op, args, mods, line, text):
        self.op, self.args, self.mods, self.line, self.text = op, args, mods, line, text


def _modifier(mods, m):
    if ":" in m:
        k, v = m.split(":", 1)
        mods[k] = int(v, 0) if k in ("offset", "offset0", "offset1") else v
    else:
        mods[m] = True


def parse_function(path: str, name: str):
    """The instructions of function ``name`` in an assembly file, and its label table."""
    instrs, labels = [], {}
    on = False
    with open(path) as fh:
        for ln, raw in enumerate(fh, 1):
            t = raw.split(";")[0].strip()
            if not on:
                on = t == name + ":"
                continue
            if t.startswith(".Lfunc_end"):
                break
            if not t:
                continue
            if t.endswith(":"):
                labels[t[:-1]] = len(instrs)
                continue
            if t.startswith("."):
                continue
            op, _, rest = t.partition(" ")
            rest = rest.strip()
            if op == "s_waitcnt":
                instrs.append(Instr(op, rest.replace("&", " ").split(), {}, ln, t))
                continue
            toks, depth, cur = [], 0, ""
            for ch in rest:  # split at commas outside brackets
                depth += ch in "[("
                depth -= ch in "])"
                if ch == "," and depth == 0:
                    toks.append(cur)
                    cur = ""
                else:
                    cur += ch
            if cur.strip():
                toks.append(cur)
            args, mods = [], {}
            for tk in toks:
                sub = tk.split()
                if not sub:
                    continue
                args.append(sub[0])
                for m in sub[1:]:
                    _modifier(mods, m)
            real = []
            for a in args:
                if ":" in a and not re.match(r"^-?\|?[sva]\[", a):
                    _modifier(mods, a)
                else:
                    real.append(a)
            instrs.append(Instr(op, [a if a.startswith(".L") else parse_operand(a) for a in real],
                                mods, ln, t))
    if not on:
        raise KeyError(f"{name} not in {path}")
    return instrs, labels


# ---------------------------------------------------------------- memory
class Memory:
    """Byte-addressed allocations.  ``add`` maps existing memory (a host buffer standing in
    for device memory) at its own address; ``alloc`` places a new buffer far from any
    host mapping."""

    def __init__(self):
        self.allocs = []   # (base, uint8 array, name), sorted by base
        self._next = 0x100000000000

    def add(self, addr, buf, name):
        self.allocs.append((addr, buf, name))
        self.allocs.sort(key=lambda t: t[0])

    def alloc(self, data, name):
        buf = np.frombuffer(bytes(data), dtype=np.uint8).copy()
        base = self._next
        self._next += (buf.size + 0x1FFFF) & ~0xFFFF
        self.add(base, buf, name)
        return base

    def find(self, addr, n):
        for base, buf, name in self.allocs:
            if base <= addr and addr + n <= base + buf.size:
                return buf, addr - base
        near = min(self.allocs, key=lambda t: min(abs(addr - t[0]), abs(addr - t[0] - t[1].size)))
        raise Fault(f"address {addr:#x} (+{n}) is outside every allocation; the nearest is "
                    f"{near[2]} at [{near[0]:#x}, {near[0] + near[1].size:#x})")

    def read(self, addr, n):
        buf, off = self.find(addr, n)
        return buf[off:off + n]

    def write(self, addr, data):
        buf, off = self.find(addr, len(data))
        buf[off:off + len(data)] = data


# ---------------------------------------------------------------- helpers
def f32(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def u32(f):
    return np.asarray(f, dtype=np.float32).view(np.uint32)


def bf16_rne(f):
    """fp32 -> bf16 bits, round to nearest even (NaN stays NaN)."""
    x = np.asarray(f, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    return np.where(np.isnan(x), 0x7FC0, r).astype(np.uint32)


def bf16_to_f32(h):
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32)


def _bits(m):
    return np.array([(int(m) >> i) & 1 for i in range(LANES)], dtype=bool)


def _mask(b):
    v = 0
    for i in np.nonzero(b)[0]:
        v |= 1 << int(i)
    return v


def _sx32(v):
    v &= M32
    return v - (1 << 32) if v & 0x80000000 else v


def _sx16(v):
    v &= 0xFFFF
    return v - (1 << 16) if v & 0x8000 else v


def _i32(x):
    return np.asarray(x, dtype=np.uint32).view(np.int32)


def _fma32(a, b, c):
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


# ---------------------------------------------------------------- wave state
class Wave:
    def __init__(self, wg, wid, priv_bytes):
        self.wg, self.wid = wg, wid
        self.s = [0] * 128
        self.v = np.zeros((512, LANES), dtype=np.uint32)
        self.a = np.zeros((256, LANES), dtype=np.uint32)
        self.exec = M64
        self.vcc = 0
        self.scc = 0
        self.m0 = 0
        self.pc = 0
        self.done = False
        self.at_barrier = False
        self.vm = []        # outstanding vector-memory ops (loads, stores, LDS copies), issue order
        self.lgkm = []      # outstanding LDS and scalar-memory ops, issue order
        self.pend = {}      # (kind, reg) -> youngest outstanding op writing it
        self.maskdef = {}   # SGPR pair / 'vcc' -> (EXEC, line) of the compare that made it
        n = max(priv_bytes, 4)
        self.priv = np.full((LANES, n), PRIV_FILL, dtype=np.uint8)
        self.priv_written = np.zeros((LANES, n), dtype=bool)

    # ---- hazards of outstanding loads
    def check_read(self, kind, idx, n=1):
        for i in range(n):
            if (kind, idx + i) in self.pend:
                raise Hazard(f"reads {kind}{idx + i} while a load into it is outstanding")

    def check_write(self, kind, idx):
        if (kind, idx) in self.pend:
            raise Hazard(f"overwrites {kind}{idx} while a load into it is outstanding")

    # ---- scalar operands
    def sget(self, o, n=None):
        n = o.n if n is None else n
        k = o.kind
        if k == "s":
            self.check_read("s", o.idx, n)
            v = 0
            for i in range(n):
                v |= self.s[o.idx + i] << (32 * i)
            return v
        if k == "i":
            return o.val & (M64 if n == 2 else M32)
        if k == "f":
            return int(u32(np.float32(o.val)))
        if k == "vcc":
            return self.vcc if n == 2 else self.vcc & M32
        if k == "vcc_lo":
            return self.vcc & M32
        if k == "vcc_hi":
            return self.vcc >> 32
        if k == "exec":
            return self.exec if n == 2 else self.exec & M32
        if k == "exec_lo":
            return self.exec & M32
        if k == "exec_hi":
            return self.exec >> 32
        if k == "m0":
            return self.m0
        if k == "scc":
            return self.scc
        raise ValueError(f"scalar read of {o}")

    def sset(self, o, val, n=None):
        n = o.n if n is None else n
        k = o.kind
        if k == "s":
            for i in range(n):
                self.check_write("s", o.idx + i)
                self.s[o.idx + i] = (val >> (32 * i)) & M32
                self.maskdef.pop(o.idx + i, None)
                self.maskdef.pop(o.idx + i - 1, None)
        elif k in ("vcc", "vcc_lo", "vcc_hi"):
            self.maskdef.pop("vcc", None)
            if k == "vcc":
                self.vcc = val & M64
            elif k == "vcc_lo":
                self.vcc = (self.vcc & (M32 << 32)) | (val & M32)
            else:
                self.vcc = (self.vcc & M32) | ((val & M32) << 32)
        elif k == "exec":
            self.exec = val & M64
        elif k == "exec_lo":
            self.exec = (self.exec & (M32 << 32)) | (val & M32)
        elif k == "exec_hi":
            self.exec = (self.exec & M32) | ((val & M32) << 32)
        elif k == "m0":
            self.m0 = val & M32
        elif k != "null":
            raise ValueError(f"scalar write of {o}")

    # ---- vector operands
    def vget(self, o):
        """Per-lane 32-bit value of an operand (uint32[64])."""
        if o.kind in ("v", "a"):
            self.check_read(o.kind, o.idx)
            return (self.v if o.kind == "v" else self.a)[o.idx].copy()
        return np.full(LANES, self.sget(o, 1) & M32, dtype=np.uint32)

    def vget64(self, o):
        if o.kind in ("v", "a"):
            arr = self.v if o.kind == "v" else self.a
            self.check_read(o.kind, o.idx, 2)
            return arr[o.idx].astype(U64) | (arr[o.idx + 1].astype(U64) << U64(32))
        if o.kind == "f":
            return np.full(LANES, struct.unpack("<Q", struct.pack("<d", o.val))[0], dtype=U64)
        return np.full(LANES, self.sget(o, 2), dtype=U64)

    def fget(self, o):
        x = np.full(LANES, np.float32(o.val), dtype=np.float32) if o.kind == "f" else f32(self.vget(o)).copy()
        if o.abs:
            x = np.abs(x)
        if o.neg:
            x = -x
        return x

    def active(self):
        return _bits(self.exec)

    def vset(self, o, val, lanes=None):
        lanes = self.active() if lanes is None else lanes
        self.check_write(o.kind, o.idx)
        arr = self.v if o.kind == "v" else self.a
        arr[o.idx][lanes] = np.asarray(val, dtype=np.uint32)[lanes] if np.ndim(val) else np.uint32(val)

    def vset64(self, o, val):
        lanes = self.active()
        val = np.asarray(val, dtype=U64)
        self.check_write(o.kind, o.idx)
        self.check_write(o.kind, o.idx + 1)
        arr = self.v if o.kind == "v" else self.a
        arr[o.idx][lanes] = (val & U64(M32)).astype(np.uint32)[lanes]
        arr[o.idx + 1][lanes] = (val >> U64(32)).astype(np.uint32)[lanes]


class WorkGroup:
    def __init__(self, machine, wg_id, nwaves):
        self.id = wg_id
        n = machine.lds_bytes
        self.lds = np.zeros(n, dtype=np.uint8)
        self.copying = np.zeros(n, dtype=np.int8)     # wave id + 1 of an unretired LDS copy
        self.rd = np.zeros((nwaves, n), dtype=bool)    # bytes read since the last barrier
        self.wr = np.zeros((nwaves, n), dtype=bool)    # bytes written since the last barrier
        self.interval = 0
        self.waves = [Wave(self, w, machine.priv_bytes) for w in range(nwaves)]
        self.lds_ops = [[] for _ in range(nwaves)]     # unretired ops touching LDS, per wave

    def touch(self, wave, addr, n, write):
        (self.wr if write else self.rd)[wave, addr:addr + n] = True

    def end_interval(self):
        """Checks the barrier interval that ends for cross-wave LDS conflicts, then carries the
        still-unretired LDS ops into the next one."""
        nw = len(self.waves)
        for a in range(nw):
            if not self.wr[a].any():
                continue
            for b in range(nw):
                if a != b:
                    clash = self.wr[a] & (self.rd[b] | self.wr[b])
                    if clash.any():
                        i = np.nonzero(clash)[0]
                        raise Hazard(f"work group {self.id}: waves {a} and {b} both touch LDS bytes "
                                     f"{i[0]}..{i[-1]} between barriers {self.interval} and "
                                     f"{self.interval + 1}, wave {a} writing")
        self.rd[:] = False
        self.wr[:] = False
        self.interval += 1
        for w in range(nw):
            for op in self.lds_ops[w]:
                for la, n, write in op["lds_span"]:
                    self.touch(w, la, n, write)


# ---------------------------------------------------------------- semantics
def _sdwa(x, sel):
    x = x.astype(np.uint32)
    if sel in (None, "DWORD"):
        return x
    if sel.startswith("WORD_"):
        return (x >> (16 * int(sel[-1]))) & 0xFFFF
    if sel.startswith("BYTE_"):
        return (x >> (8 * int(sel[-1]))) & 0xFF
    raise ValueError(sel)


def _mfma_layout(m):
    """Index arrays of an MxMxK MFMA's operands (K = 8 * 64 / M).  A: lane l holds row
    l % M, k = 8 (l / M) .. +7; B: column l % M, the same k.  D: for 32x32, register r of
    lane l is row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32; for 16x16, row
    4 (l / 16) + r, column l % 16."""
    lanes = np.arange(LANES)
    rows = np.repeat(lanes % m, 8)
    ks = ((8 * (lanes // m))[:, None] + np.arange(8)).reshape(-1)
    if m == 32:
        drow = np.array([[8 * (r // 4) + 4 * (l // 32) + r % 4 for l in range(LANES)] for r in range(16)])
    else:
        drow = np.array([[4 * (l // 16) + r for l in range(LANES)] for r in range(4)])
    return rows, ks, drow, lanes % m


_MFMA_LAYOUT = {32: _mfma_layout(32), 16: _mfma_layout(16)}


class Semantics:
    """One handler per opcode: ``op_<mnemonic>(wave, instr)``."""

    def __init__(self, machine):
        self.m = machine

    # ------------------------------------------------ small helpers
    def S(self, w, o, n=None):
        return w.sget(o, n)

    def V(self, w, o):
        return w.vget(o)

    def F(self, w, o):
        return w.fget(o)

    def WS(self, w, o, val, n=None):
        w.sset(o, val & (M64 if (n or o.n) == 2 else M32), n)

    def WV(self, w, o, vals):
        w.vset(o, vals)

    def WF(self, w, o, f):
        w.vset(o, u32(np.asarray(f, dtype=np.float32)))

    def lane_mask(self, w, b):
        return _mask(np.asarray(b) & w.active())

    def made_under(self, w, o, i):
        """Records the EXEC a compare's lane mask was made under."""
        key = o.idx if o.kind == "s" and o.n == 2 else ("vcc" if o.kind == "vcc" else None)
        if key is not None:
            w.maskdef[key] = (w.exec, i.line)

    def used_under(self, w, o, i, what):
        key = o.idx if o.kind == "s" and o.n == 2 else ("vcc" if o.kind == "vcc" else None)
        rec = w.maskdef.get(key) if key is not None else None
        if rec is None or not (w.exec & ~rec[0]):
            return
        self.m.note_once(("mask", rec[1], i.line),
                         f"lane mask {o} made at line {rec[1]} under EXEC {rec[0]:016x} is used by {what} "
                         f"at line {i.line} ({i.text}) under EXEC {w.exec:016x}")

    # ------------------------------------------------ SALU
    def _s2(self, w, i, f, n=1):
        r = f(self.S(w, i.args[1], n), self.S(w, i.args[2], n)) & (M64 if n == 2 else M32)
        self.WS(w, i.args[0], r, n)
        w.scc = int(r != 0)

    def op_s_mov_b32(self, w, i): self.WS(w, i.args[0], self.S(w, i.args[1], 1), 1)
    def op_s_mov_b64(self, w, i): self.WS(w, i.args[0], self.S(w, i.args[1], 2), 2)
    def op_s_movk_i32(self, w, i): self.WS(w, i.args[0], _sx16(i.args[1].val) & M32, 1)

    def op_s_cselect_b32(self, w, i):
        self.WS(w, i.args[0], self.S(w, i.args[1 if w.scc else 2], 1), 1)

    def op_s_cselect_b64(self, w, i):
        self.WS(w, i.args[0], self.S(w, i.args[1 if w.scc else 2], 2), 2)

    def op_s_add_u32(self, w, i):
        r = self.S(w, i.args[1], 1) + self.S(w, i.args[2], 1)
        self.WS(w, i.args[0], r, 1)
        w.scc = int(r > M32)

    def op_s_addc_u32(self, w, i):
        r = self.S(w, i.args[1], 1) + self.S(w, i.args[2], 1) + w.scc
        self.WS(w, i.args[0], r, 1)
        w.scc = int(r > M32)

    def op_s_sub_u32(self, w, i):
        a, b = self.S(w, i.args[1], 1), self.S(w, i.args[2], 1)
        self.WS(w, i.args[0], a - b, 1)
        w.scc = int(b > a)

    def op_s_subb_u32(self, w, i):
        a, b, c = self.S(w, i.args[1], 1), self.S(w, i.args[2], 1), w.scc
        self.WS(w, i.args[0], a - b - c, 1)
        w.scc = int(b + c > a)

    def _add_i32(self, w, dst, a, b):
        r = _sx32(a) + _sx32(b)
        self.WS(w, dst, r, 1)
        w.scc = int(not -(1 << 31) <= r < (1 << 31))

    def op_s_add_i32(self, w, i): self._add_i32(w, i.args[0], self.S(w, i.args[1], 1), self.S(w, i.args[2], 1))
    def op_s_addk_i32(self, w, i): self._add_i32(w, i.args[0], self.S(w, i.args[0], 1), _sx16(i.args[1].val))

    def op_s_sub_i32(self, w, i):
        r = _sx32(self.S(w, i.args[1], 1)) - _sx32(self.S(w, i.args[2], 1))
        self.WS(w, i.args[0], r, 1)
        w.scc = int(not -(1 << 31) <= r < (1 << 31))

    def op_s_mul_i32(self, w, i):
        self.WS(w, i.args[0], _sx32(self.S(w, i.args[1], 1)) * _sx32(self.S(w, i.args[2], 1)), 1)

    def op_s_mul_hi_u32(self, w, i):
        self.WS(w, i.args[0], (self.S(w, i.args[1], 1) * self.S(w, i.args[2], 1)) >> 32, 1)

    def op_s_mul_hi_i32(self, w, i):
        self.WS(w, i.args[0], (_sx32(self.S(w, i.args[1], 1)) * _sx32(self.S(w, i.args[2], 1))) >> 32, 1)

    def _minmax(self, w, i, signed, pick_min):
        a, b = self.S(w, i.args[1], 1), self.S(w, i.args[2], 1)
        x, y = (_sx32(a), _sx32(b)) if signed else (a, b)
        take_a = x < y if pick_min else x > y
        self.WS(w, i.args[0], a if take_a else b, 1)
        w.scc = int(take_a)

    def op_s_min_i32(self, w, i): self._minmax(w, i, True, True)
    def op_s_max_i32(self, w, i): self._minmax(w, i, True, False)
    def op_s_min_u32(self, w, i): self._minmax(w, i, False, True)
    def op_s_max_u32(self, w, i): self._minmax(w, i, False, False)

    def op_s_abs_i32(self, w, i):
        r = abs(_sx32(self.S(w, i.args[1], 1))) & M32
        self.WS(w, i.args[0], r, 1)
        w.scc = int(r != 0)

    def op_s_and_b32(self, w, i): self._s2(w, i, lambda a, b: a & b)
    def op_s_or_b32(self, w, i): self._s2(w, i, lambda a, b: a | b)
    def op_s_xor_b32(self, w, i): self._s2(w, i, lambda a, b: a ^ b)
    def op_s_andn2_b32(self, w, i): self._s2(w, i, lambda a, b: a & ~b)
    def op_s_or_b64(self, w, i): self._s2(w, i, lambda a, b: a | b, 2)
    def op_s_xor_b64(self, w, i): self._s2(w, i, lambda a, b: a ^ b, 2)
    def op_s_andn2_b64(self, w, i): self._s2(w, i, lambda a, b: a & ~b, 2)
    def op_s_orn2_b64(self, w, i): self._s2(w, i, lambda a, b: a | ~b, 2)
    def op_s_nor_b64(self, w, i): self._s2(w, i, lambda a, b: ~(a | b), 2)
    def op_s_lshl_b32(self, w, i): self._s2(w, i, lambda a, b: a << (b & 31))
    def op_s_lshr_b32(self, w, i): self._s2(w, i, lambda a, b: a >> (b & 31))
    def op_s_ashr_i32(self, w, i): self._s2(w, i, lambda a, b: _sx32(a) >> (b & 31))

    def op_s_and_b64(self, w, i):
        a, b = i.args[1], i.args[2]
        if a.kind == "exec":
            self.used_under(w, b, i, "s_and_b64 with exec")
        elif b.kind == "exec":
            self.used_under(w, a, i, "s_and_b64 with exec")
        self._s2(w, i, lambda x, y: x & y, 2)

    def _shift64(self, w, i, f):
        r = f(self.S(w, i.args[1], 2), self.S(w, i.args[2], 1) & 63) & M64
        self.WS(w, i.args[0], r, 2)
        w.scc = int(r != 0)

    def op_s_lshl_b64(self, w, i): self._shift64(w, i, lambda a, b: a << b)
    def op_s_lshr_b64(self, w, i): self._shift64(w, i, lambda a, b: a >> b)
    def op_s_ashr_i64(self, w, i): self._shift64(w, i, lambda a, b: (a - (1 << 64) if a >> 63 else a) >> b)

    def _lshl_add(self, w, i, n):
        r = (self.S(w, i.args[1], 1) << n) + self.S(w, i.args[2], 1)
        self.WS(w, i.args[0], r, 1)
        w.scc = int(r > M32)

    def op_s_lshl1_add_u32(self, w, i): self._lshl_add(w, i, 1)
    def op_s_lshl2_add_u32(self, w, i): self._lshl_add(w, i, 2)
    def op_s_lshl3_add_u32(self, w, i): self._lshl_add(w, i, 3)
    def op_s_lshl4_add_u32(self, w, i): self._lshl_add(w, i, 4)

    def op_s_not_b32(self, w, i):
        r = ~self.S(w, i.args[1], 1) & M32
        self.WS(w, i.args[0], r, 1)
        w.scc = int(r != 0)

    def op_s_not_b64(self, w, i):
        r = ~self.S(w, i.args[1], 2) & M64
        self.WS(w, i.args[0], r, 2)
        w.scc = int(r != 0)

    def op_s_bfe_u32(self, w, i):
        a, b = self.S(w, i.args[1], 1), self.S(w, i.args[2], 1)
        off, wid = b & 31, (b >> 16) & 127
        r = (a >> off) & ((1 << wid) - 1) if wid else 0
        self.WS(w, i.args[0], r, 1)
        w.scc = int(r != 0)

    def op_s_bfe_i32(self, w, i):
        a, b = self.S(w, i.args[1], 1), self.S(w, i.args[2], 1)
        off, wid = b & 31, (b >> 16) & 127
        r = 0
        if wid:
            r = (a >> off) & ((1 << wid) - 1)
            if wid < 32 and (r >> (wid - 1)) & 1:
                r -= 1 << wid
        self.WS(w, i.args[0], r, 1)
        w.scc = int((r & M32) != 0)

    def op_s_bfm_b32(self, w, i):
        a, b = self.S(w, i.args[1], 1), self.S(w, i.args[2], 1)
        self.WS(w, i.args[0], ((1 << (a & 31)) - 1) << (b & 31), 1)

    def op_s_brev_b32(self, w, i):
        self.WS(w, i.args[0], int("{:032b}".format(self.S(w, i.args[1], 1))[::-1], 2), 1)

    def op_s_ff1_i32_b32(self, w, i):
        a = self.S(w, i.args[1], 1)
        self.WS(w, i.args[0], (a & -a).bit_length() - 1 if a else M32, 1)

    def op_s_ff1_i32_b64(self, w, i):
        a = self.S(w, i.args[1], 2)
        self.WS(w, i.args[0], (a & -a).bit_length() - 1 if a else M32, 1)

    def op_s_flbit_i32_b32(self, w, i):
        a = self.S(w, i.args[1], 1)
        self.WS(w, i.args[0], 32 - a.bit_length() if a else M32, 1)

    def op_s_bcnt1_i32_b32(self, w, i):
        r = bin(self.S(w, i.args[1], 1)).count("1")
        self.WS(w, i.args[0], r, 1)
        w.scc = int(r != 0)

    def op_s_bcnt1_i32_b64(self, w, i):
        r = bin(self.S(w, i.args[1], 2)).count("1")
        self.WS(w, i.args[0], r, 1)
        w.scc = int(r != 0)

    def op_s_sext_i32_i16(self, w, i): self.WS(w, i.args[0], _sx16(self.S(w, i.args[1], 1)), 1)

    def op_s_pack_ll_b32_b16(self, w, i):
        a, b = self.S(w, i.args[1], 1), self.S(w, i.args[2], 1)
        self.WS(w, i.args[0], (a & 0xFFFF) | ((b & 0xFFFF) << 16), 1)

    def _scmp(self, w, i, f, signed, n=1):
        a, b = self.S(w, i.args[0], n), self.S(w, i.args[1], n)
        if signed:
            a, b = _sx32(a), _sx32(b)
        w.scc = int(f(a, b))

    def op_s_bitcmp0_b32(self, w, i):
        w.scc = int(((self.S(w, i.args[0], 1) >> (self.S(w, i.args[1], 1) & 31)) & 1) == 0)

    def op_s_bitcmp1_b32(self, w, i):
        w.scc = int(((self.S(w, i.args[0], 1) >> (self.S(w, i.args[1], 1) & 31)) & 1) == 1)

    def _saveexec(self, w, i, f, name):
        self.used_under(w, i.args[1], i, name)
        old = w.exec
        w.exec = f(self.S(w, i.args[1], 2), old) & M64
        self.WS(w, i.args[0], old, 2)
        w.scc = int(w.exec != 0)

    def op_s_and_saveexec_b64(self, w, i): self._saveexec(w, i, lambda s, e: s & e, "s_and_saveexec_b64")
    def op_s_or_saveexec_b64(self, w, i): self._saveexec(w, i, lambda s, e: s | e, "s_or_saveexec_b64")
    def op_s_xor_saveexec_b64(self, w, i): self._saveexec(w, i, lambda s, e: s ^ e, "s_xor_saveexec_b64")
    def op_s_andn2_saveexec_b64(self, w, i): self._saveexec(w, i, lambda s, e: s & ~e, "s_andn2_saveexec_b64")

    # ------------------------------------------------ program flow
    def _jump(self, w, i):
        w.pc = self.m.labels[i.args[0]]

    def op_s_branch(self, w, i): self._jump(w, i)

    def op_s_cbranch_scc0(self, w, i):
        if not w.scc:
            self._jump(w, i)

    def op_s_cbranch_scc1(self, w, i):
        if w.scc:
            self._jump(w, i)

    def op_s_cbranch_vccz(self, w, i):
        if w.vcc == 0:
            self._jump(w, i)

    def op_s_cbranch_vccnz(self, w, i):
        if w.vcc != 0:
            self._jump(w, i)

    def op_s_cbranch_execz(self, w, i):
        if w.exec == 0:
            self._jump(w, i)

    def op_s_cbranch_execnz(self, w, i):
        if w.exec != 0:
            self._jump(w, i)

    def op_s_endpgm(self, w, i):
        self.m.retire(w, "vm", 0)
        self.m.retire(w, "lgkm", 0)
        w.done = True

    def op_s_barrier(self, w, i): w.at_barrier = True
    def op_s_nop(self, w, i): pass
    def op_s_setprio(self, w, i): pass
    def op_s_sleep(self, w, i): pass

    def op_s_waitcnt(self, w, i):
        for t in i.args:
            mm = re.match(r"(vmcnt|lgkmcnt|expcnt)\((\d+)\)", t)
            if not mm:
                raise ValueError(i.text)
            n = int(mm.group(2))
            if mm.group(1) == "vmcnt":
                self.m.retire(w, "vm", n)
            elif mm.group(1) == "lgkmcnt":
                if n > 0 and any(op["smem"] for op in w.lgkm):
                    self.m.note_once(("smem", i.line), f"line {i.line}: lgkmcnt({n}) with scalar loads "
                                     "outstanding (they may complete out of order)")
                self.m.retire(w, "lgkm", n)

    # ------------------------------------------------ scalar memory
    def _sload(self, w, i, n):
        base = self.S(w, i.args[1], 2)
        off = self.S(w, i.args[2], 1) if len(i.args) > 2 else 0
        data = self.m.mem.read((base + off) & ~3, 4 * n).view(np.uint32).copy()
        dst = i.args[0]
        for k in range(n):
            w.check_write("s", dst.idx + k)
        op = {"smem": True, "writes": [(("s", dst.idx + k), int(data[k]), None) for k in range(n)]}
        w.lgkm.append(op)
        for k in range(n):
            w.pend[("s", dst.idx + k)] = op

    def op_s_load_dword(self, w, i): self._sload(w, i, 1)
    def op_s_load_dwordx2(self, w, i): self._sload(w, i, 2)
    def op_s_load_dwordx4(self, w, i): self._sload(w, i, 4)
    def op_s_load_dwordx8(self, w, i): self._sload(w, i, 8)
    def op_s_load_dwordx16(self, w, i): self._sload(w, i, 16)

    # ------------------------------------------------ VALU integer
    def _v2(self, w, i, f):
        a, b = self.V(w, i.args[1]).astype(U64), self.V(w, i.args[2]).astype(U64)
        self.WV(w, i.args[0], (f(a, b) & U64(M32)).astype(U32))

    def _v3(self, w, i, f):
        a, b, c = (self.V(w, x).astype(U64) for x in i.args[1:4])
        self.WV(w, i.args[0], (f(a, b, c) & U64(M32)).astype(U32))

    def op_v_mov_b32_e32(self, w, i): self.WV(w, i.args[0], self.V(w, i.args[1]))
    op_v_mov_b32_e64 = op_v_mov_b32_e32
    def op_v_mov_b64_e32(self, w, i): w.vset64(i.args[0], w.vget64(i.args[1]))
    def op_v_add_u32_e32(self, w, i): self._v2(w, i, lambda a, b: a + b)
    op_v_add_u32_e64 = op_v_add_u32_e32
    def op_v_sub_u32_e32(self, w, i): self._v2(w, i, lambda a, b: a - b)
    def op_v_subrev_u32_e32(self, w, i): self._v2(w, i, lambda a, b: b - a)

    def _sub_clamp(self, w, i, rev):
        a, b = self.V(w, i.args[1]).astype(np.int64), self.V(w, i.args[2]).astype(np.int64)
        r = b - a if rev else a - b
        if i.mods.get("clamp"):
            r = np.maximum(r, 0)
        self.WV(w, i.args[0], (r & M32).astype(U32))

    def op_v_sub_u32_e64(self, w, i): self._sub_clamp(w, i, False)
    def op_v_subrev_u32_e64(self, w, i): self._sub_clamp(w, i, True)
    def op_v_add3_u32(self, w, i): self._v3(w, i, lambda a, b, c: a + b + c)
    def op_v_add_lshl_u32(self, w, i): self._v3(w, i, lambda a, b, c: ((a + b) & U64(M32)) << (c & U64(31)))
    def op_v_lshl_add_u32(self, w, i): self._v3(w, i, lambda a, b, c: ((a << (b & U64(31))) & U64(M32)) + c)
    def op_v_lshl_or_b32(self, w, i): self._v3(w, i, lambda a, b, c: ((a << (b & U64(31))) & U64(M32)) | c)
    def op_v_and_or_b32(self, w, i): self._v3(w, i, lambda a, b, c: (a & b) | c)
    def op_v_or3_b32(self, w, i): self._v3(w, i, lambda a, b, c: a | b | c)
    def op_v_xor3_b32(self, w, i): self._v3(w, i, lambda a, b, c: a ^ b ^ c)
    def op_v_xad_u32(self, w, i): self._v3(w, i, lambda a, b, c: (a ^ b) + c)
    def op_v_bfi_b32(self, w, i): self._v3(w, i, lambda a, b, c: (a & b) | (~a & c))
    def op_v_alignbit_b32(self, w, i): self._v3(w, i, lambda a, b, c: ((a << U64(32)) | b) >> (c & U64(31)))
    def op_v_alignbyte_b32(self, w, i): self._v3(w, i, lambda a, b, c: ((a << U64(32)) | b) >> (U64(8) * (c & U64(3))))
    def op_v_and_b32_e32(self, w, i): self._v2(w, i, lambda a, b: a & b)
    op_v_and_b32_e64 = op_v_and_b32_e32
    def op_v_or_b32_e32(self, w, i): self._v2(w, i, lambda a, b: a | b)
    op_v_or_b32_e64 = op_v_or_b32_e32
    def op_v_xor_b32_e32(self, w, i): self._v2(w, i, lambda a, b: a ^ b)
    op_v_xor_b32_e64 = op_v_xor_b32_e32
    def op_v_not_b32_e32(self, w, i): self.WV(w, i.args[0], ~self.V(w, i.args[1]))
    def op_v_lshlrev_b32_e32(self, w, i): self._v2(w, i, lambda a, b: b << (a & U64(31)))
    op_v_lshlrev_b32_e64 = op_v_lshlrev_b32_e32
    def op_v_lshrrev_b32_e32(self, w, i): self._v2(w, i, lambda a, b: b >> (a & U64(31)))
    op_v_lshrrev_b32_e64 = op_v_lshrrev_b32_e32
    def op_v_mul_lo_u32(self, w, i): self._v2(w, i, lambda a, b: a * b)
    def op_v_add_u16_e32(self, w, i): self._v2(w, i, lambda a, b: (a + b) & U64(0xFFFF))
    def op_v_sub_u16_e32(self, w, i): self._v2(w, i, lambda a, b: (a - b) & U64(0xFFFF))

    def op_v_ashrrev_i32_e32(self, w, i):
        a, b = self.V(w, i.args[1]), _i32(self.V(w, i.args[2]))
        self.WV(w, i.args[0], (b >> (a & 31).astype(I32)).view(U32))
    op_v_ashrrev_i32_e64 = op_v_ashrrev_i32_e32

    def op_v_bfe_u32(self, w, i):
        a, b, c = self.V(w, i.args[1]), self.V(w, i.args[2]) & 31, self.V(w, i.args[3]) & 31
        r = (a.astype(U64) >> b.astype(U64)) & ((U64(1) << c.astype(U64)) - U64(1))
        self.WV(w, i.args[0], r.astype(U32))

    def op_v_bfrev_b32_e32(self, w, i):
        self.WV(w, i.args[0], np.array([int("{:032b}".format(int(x))[::-1], 2) for x in self.V(w, i.args[1])],
                                       dtype=U32))

    def op_v_bcnt_u32_b32(self, w, i):
        pc = np.array([bin(int(x)).count("1") for x in self.V(w, i.args[1])], dtype=U32)
        self.WV(w, i.args[0], pc + self.V(w, i.args[2]))

    def op_v_ffbh_u32_e32(self, w, i):
        self.WV(w, i.args[0], np.array([32 - int(x).bit_length() if x else M32 for x in self.V(w, i.args[1])],
                                       dtype=U32))

    def op_v_bitop3_b32(self, w, i):
        # result bit = table bit (s0 << 2 | s1 << 1 | s2)
        a, b, c = (self.V(w, x).astype(U64) for x in i.args[1:4])
        t = int(i.mods["bitop3"], 0)
        r = np.zeros(LANES, dtype=U64)
        for k in range(8):
            if (t >> k) & 1:
                r |= (a if k & 4 else ~a) & (b if k & 2 else ~b) & (c if k & 1 else ~c)
        self.WV(w, i.args[0], (r & U64(M32)).astype(U32))

    def _vminmax(self, w, i, f, signed):
        a, b = self.V(w, i.args[1]), self.V(w, i.args[2])
        if signed:
            self.WV(w, i.args[0], f(_i32(a), _i32(b)).view(U32))
        else:
            self.WV(w, i.args[0], f(a, b))

    def op_v_max_i32_e32(self, w, i): self._vminmax(w, i, np.maximum, True)
    op_v_max_i32_e64 = op_v_max_i32_e32
    def op_v_min_i32_e32(self, w, i): self._vminmax(w, i, np.minimum, True)
    op_v_min_i32_e64 = op_v_min_i32_e32
    def op_v_max_u32_e32(self, w, i): self._vminmax(w, i, np.maximum, False)
    op_v_max_u32_e64 = op_v_max_u32_e32
    def op_v_min_u32_e32(self, w, i): self._vminmax(w, i, np.minimum, False)
    op_v_min_u32_e64 = op_v_min_u32_e32

    def op_v_max3_i32(self, w, i):
        a, b, c = (_i32(self.V(w, x)) for x in i.args[1:4])
        self.WV(w, i.args[0], np.maximum(np.maximum(a, b), c).view(U32))

    def op_v_min3_i32(self, w, i):
        a, b, c = (_i32(self.V(w, x)) for x in i.args[1:4])
        self.WV(w, i.args[0], np.minimum(np.minimum(a, b), c).view(U32))

    def op_v_med3_i32(self, w, i):
        a, b, c = (_i32(self.V(w, x)).astype(np.int64) for x in i.args[1:4])
        r = np.maximum(np.minimum(a, b), np.minimum(np.maximum(a, b), c))
        self.WV(w, i.args[0], (r & M32).astype(U32))

    def op_v_mul_hi_u32(self, w, i):
        a, b = self.V(w, i.args[1]), self.V(w, i.args[2])
        self.WV(w, i.args[0], np.array([(int(x) * int(y)) >> 32 for x, y in zip(a, b)], dtype=U32))

    def op_v_mad_u64_u32(self, w, i):
        a, b = self.V(w, i.args[2]), self.V(w, i.args[3])
        c = w.vget64(i.args[4])
        r = [int(x) * int(y) + int(z) for x, y, z in zip(a, b, c)]
        w.vset64(i.args[0], np.array([x & M64 for x in r], dtype=U64))
        self.WS(w, i.args[1], self.lane_mask(w, np.array([x >> 64 != 0 for x in r])), 2)

    def op_v_mad_i64_i32(self, w, i):
        a, b = _i32(self.V(w, i.args[2])), _i32(self.V(w, i.args[3]))
        c = [int(z) - (1 << 64) if int(z) >> 63 else int(z) for z in w.vget64(i.args[4])]
        r = [int(x) * int(y) + z for x, y, z in zip(a, b, c)]
        w.vset64(i.args[0], np.array([x & M64 for x in r], dtype=U64))
        self.WS(w, i.args[1], self.lane_mask(w, np.array([not -(1 << 63) <= x < (1 << 63) for x in r])), 2)

    def op_v_lshl_add_u64(self, w, i):
        sh = self.V(w, i.args[2]).astype(U64) & U64(63)
        w.vset64(i.args[0], (w.vget64(i.args[1]) << sh) + w.vget64(i.args[3]))

    def op_v_lshlrev_b64(self, w, i):
        w.vset64(i.args[0], w.vget64(i.args[2]) << (self.V(w, i.args[1]).astype(U64) & U64(63)))

    def op_v_lshrrev_b64(self, w, i):
        w.vset64(i.args[0], w.vget64(i.args[2]) >> (self.V(w, i.args[1]).astype(U64) & U64(63)))

    def op_v_mbcnt_lo_u32_b32(self, w, i):
        mk = self.S(w, i.args[1], 1)
        r = np.array([bin(mk & ((1 << min(l, 32)) - 1)).count("1") for l in range(LANES)], dtype=U32)
        self.WV(w, i.args[0], r + self.V(w, i.args[2]))

    def op_v_mbcnt_hi_u32_b32(self, w, i):
        mk = self.S(w, i.args[1], 1)
        r = np.array([bin(mk & ((1 << max(l - 32, 0)) - 1)).count("1") for l in range(LANES)], dtype=U32)
        self.WV(w, i.args[0], r + self.V(w, i.args[2]))

    # carry forms: vdst, carry-out, src0, src1 [, carry-in]
    def _carry(self, w, i, sub, rev, cin):
        a = self.V(w, i.args[2]).astype(np.int64)
        b = self.V(w, i.args[3]).astype(np.int64)
        if rev:
            a, b = b, a
        c = _bits(self.S(w, i.args[4], 2)).astype(np.int64) if cin else 0
        r = a - b - c if sub else a + b + c
        self.WV(w, i.args[0], (r & M32).astype(U32))
        self.WS(w, i.args[1], self.lane_mask(w, r < 0 if sub else r > M32), 2)

    def op_v_add_co_u32_e32(self, w, i): self._carry(w, i, False, False, False)
    op_v_add_co_u32_e64 = op_v_add_co_u32_e32
    def op_v_addc_co_u32_e32(self, w, i): self._carry(w, i, False, False, True)
    op_v_addc_co_u32_e64 = op_v_addc_co_u32_e32
    def op_v_sub_co_u32_e32(self, w, i): self._carry(w, i, True, False, False)
    op_v_sub_co_u32_e64 = op_v_sub_co_u32_e32
    def op_v_subrev_co_u32_e32(self, w, i): self._carry(w, i, True, True, False)
    op_v_subrev_co_u32_e64 = op_v_subrev_co_u32_e32
    def op_v_subb_co_u32_e32(self, w, i): self._carry(w, i, True, False, True)
    op_v_subb_co_u32_e64 = op_v_subb_co_u32_e32
    def op_v_subbrev_co_u32_e32(self, w, i): self._carry(w, i, True, True, True)
    op_v_subbrev_co_u32_e64 = op_v_subbrev_co_u32_e32

    def op_v_cndmask_b32_e32(self, w, i):
        self.used_under(w, Operand("vcc"), i, "v_cndmask_b32_e32")
        sel = _bits(w.vcc)
        self.WV(w, i.args[0], np.where(sel, self.V(w, i.args[2]), self.V(w, i.args[1])))

    def op_v_cndmask_b32_e64(self, w, i):
        self.used_under(w, i.args[3], i, "v_cndmask_b32_e64")
        sel = _bits(self.S(w, i.args[3], 2))
        a0, a1 = i.args[1], i.args[2]
        if a0.abs or a0.neg or a1.abs or a1.neg:
            a, b = u32(self.F(w, a0)), u32(self.F(w, a1))
        else:
            a, b = self.V(w, a0), self.V(w, a1)
        self.WV(w, i.args[0], np.where(sel, b, a))

    # ------------------------------------------------ compares
    def _vcmp(self, w, i, f, kind, sdwa=False):
        x, y = i.args[1], i.args[2]
        if kind == "u32":
            a, b = self.V(w, x), self.V(w, y)
        elif kind == "i32":
            a, b = _i32(self.V(w, x)), _i32(self.V(w, y))
        elif kind == "u16":
            a = _sdwa(self.V(w, x), i.mods.get("src0_sel")) & 0xFFFF
            b = _sdwa(self.V(w, y), i.mods.get("src1_sel")) & 0xFFFF
        elif kind == "u64":
            a, b = w.vget64(x), w.vget64(y)
        elif kind == "i64":
            a, b = w.vget64(x).view(np.int64), w.vget64(y).view(np.int64)
        else:
            a, b = self.F(w, x), self.F(w, y)
        self.WS(w, i.args[0], self.lane_mask(w, f(a, b)), 2)
        self.made_under(w, i.args[0], i)

    # ------------------------------------------------ VALU float
    def _f2(self, w, i, f):
        with np.errstate(all="ignore"):
            self.WF(w, i.args[0], f(self.F(w, i.args[1]), self.F(w, i.args[2])).astype(np.float32))

    def _f1(self, w, i, f):
        with np.errstate(all="ignore"):
            self.WF(w, i.args[0], f(self.F(w, i.args[1])).astype(np.float32))

    def op_v_mul_f32_e32(self, w, i): self._f2(w, i, lambda a, b: a * b)
    op_v_mul_f32_e64 = op_v_mul_f32_e32
    def op_v_add_f32_e32(self, w, i): self._f2(w, i, lambda a, b: a + b)
    op_v_add_f32_e64 = op_v_add_f32_e32
    def op_v_sub_f32_e32(self, w, i): self._f2(w, i, lambda a, b: a - b)
    op_v_sub_f32_e64 = op_v_sub_f32_e32
    def op_v_subrev_f32_e32(self, w, i): self._f2(w, i, lambda a, b: b - a)
    op_v_subrev_f32_e64 = op_v_subrev_f32_e32
    def op_v_max_f32_e32(self, w, i): self._f2(w, i, np.fmax)
    op_v_max_f32_e64 = op_v_max_f32_e32
    def op_v_min_f32_e32(self, w, i): self._f2(w, i, np.fmin)
    op_v_min_f32_e64 = op_v_min_f32_e32

    def op_v_max3_f32(self, w, i):
        a, b, c = (self.F(w, x) for x in i.args[1:4])
        self.WF(w, i.args[0], np.fmax(np.fmax(a, b), c))

    def op_v_min3_f32(self, w, i):
        a, b, c = (self.F(w, x) for x in i.args[1:4])
        self.WF(w, i.args[0], np.fmin(np.fmin(a, b), c))

    def op_v_fma_f32(self, w, i):
        with np.errstate(all="ignore"):
            self.WF(w, i.args[0], _fma32(*(self.F(w, x) for x in i.args[1:4])))

    def op_v_fmac_f32_e32(self, w, i):
        with np.errstate(all="ignore"):
            self.WF(w, i.args[0], _fma32(self.F(w, i.args[1]), self.F(w, i.args[2]), self.F(w, i.args[0])))
    op_v_fmac_f32_e64 = op_v_fmac_f32_e32

    def op_v_fmamk_f32(self, w, i):  # d = s0 * K + s1
        with np.errstate(all="ignore"):
            self.WF(w, i.args[0], _fma32(self.F(w, i.args[1]), self.F(w, i.args[2]), self.F(w, i.args[3])))

    def op_v_fmaak_f32(self, w, i):  # d = s0 * s1 + K
        with np.errstate(all="ignore"):
            self.WF(w, i.args[0], _fma32(self.F(w, i.args[1]), self.F(w, i.args[2]), self.F(w, i.args[3])))

    def op_v_fma_mix_f32(self, w, i):
        """fp32 FMA whose sources are fp16 halves (op_sel_hi set: op_sel picks the half) or fp32."""
        def sel(s):
            return [int(x) for x in s.strip("[]").split(",")] if s else [0, 0, 0]
        osel, ohi = sel(i.mods.get("op_sel")), sel(i.mods.get("op_sel_hi"))
        vals = []
        for k, o in enumerate(i.args[1:4]):
            if ohi[k]:
                raw = self.V(w, o)
                half = (raw >> 16) if osel[k] else (raw & 0xFFFF)
                x = half.astype(np.uint16).view(np.float16).astype(np.float32)
                if o.abs:
                    x = np.abs(x)
                if o.neg:
                    x = -x
            else:
                x = self.F(w, o)
            vals.append(x)
        with np.errstate(all="ignore"):
            self.WF(w, i.args[0], _fma32(*vals))

    def op_v_exp_f32_e32(self, w, i): self._f1(w, i, np.exp2)
    def op_v_log_f32_e32(self, w, i): self._f1(w, i, np.log2)
    def op_v_rcp_f32_e32(self, w, i): self._f1(w, i, lambda a: np.float32(1.0) / a)
    op_v_rcp_iflag_f32_e32 = op_v_rcp_f32_e32
    def op_v_sqrt_f32_e32(self, w, i): self._f1(w, i, np.sqrt)
    def op_v_trunc_f32_e32(self, w, i): self._f1(w, i, np.trunc)
    def op_v_floor_f32_e32(self, w, i): self._f1(w, i, np.floor)
    def op_v_rndne_f32_e32(self, w, i): self._f1(w, i, np.rint)

    def op_v_ldexp_f32(self, w, i):
        with np.errstate(all="ignore"):
            self.WF(w, i.args[0], np.ldexp(self.F(w, i.args[1]), _i32(self.V(w, i.args[2]))).astype(np.float32))

    # IEEE division: modelled without the range scaling (its flag stays 0), which matters
    # only for operands near the ends of the exponent range; the fixup handles specials.
    def op_v_div_scale_f32(self, w, i):
        self.WF(w, i.args[0], self.F(w, i.args[2]))
        self.WS(w, i.args[1], 0, 2)

    def op_v_div_fmas_f32(self, w, i):
        with np.errstate(all="ignore"):
            self.WF(w, i.args[0], _fma32(*(self.F(w, x) for x in i.args[1:4])))

    def op_v_div_fixup_f32(self, w, i):
        q, den, num = (self.F(w, x) for x in i.args[1:4])
        with np.errstate(all="ignore"):
            exact = (num.astype(np.float64) / den.astype(np.float64)).astype(np.float32)
        special = ~np.isfinite(den) | (den == 0) | ~np.isfinite(num) | ~np.isfinite(q)
        self.WF(w, i.args[0], np.where(special, exact, q))

    def op_v_cvt_f32_u32_e32(self, w, i): self.WF(w, i.args[0], self.V(w, i.args[1]).astype(np.float32))
    def op_v_cvt_f32_i32_e32(self, w, i): self.WF(w, i.args[0], _i32(self.V(w, i.args[1])).astype(np.float32))

    def op_v_cvt_u32_f32_e32(self, w, i):
        a = self.F(w, i.args[1]).astype(np.float64)
        a = np.where(np.isnan(a), 0, np.clip(np.trunc(a), 0, M32))
        self.WV(w, i.args[0], a.astype(np.uint64).astype(U32))

    def op_v_cvt_i32_f32_e32(self, w, i):
        a = self.F(w, i.args[1]).astype(np.float64)
        a = np.where(np.isnan(a), 0, np.clip(np.trunc(a), -2 ** 31, 2 ** 31 - 1))
        self.WV(w, i.args[0], a.astype(np.int64).astype(np.int32).view(U32))

    def op_v_cvt_pk_bf16_f32(self, w, i):
        self.WV(w, i.args[0], bf16_rne(self.F(w, i.args[1])) | (bf16_rne(self.F(w, i.args[2])) << 16))

    def op_v_cvt_pk_f16_f32(self, w, i):
        with np.errstate(all="ignore"):
            lo = self.F(w, i.args[1]).astype(np.float16).view(np.uint16).astype(U32)
            hi = self.F(w, i.args[2]).astype(np.float16).view(np.uint16).astype(U32)
        self.WV(w, i.args[0], lo | (hi << 16))

    def op_v_cvt_f32_f16_e32(self, w, i):
        self.WF(w, i.args[0], (self.V(w, i.args[1]) & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float32))

    # ------------------------------------------------ cross-lane
    def op_v_readlane_b32(self, w, i):
        o = i.args[1]
        w.check_read(o.kind, o.idx)
        lane = self.S(w, i.args[2], 1) & 63
        self.WS(w, i.args[0], int((w.v if o.kind == "v" else w.a)[o.idx][lane]), 1)

    def op_v_readfirstlane_b32(self, w, i):
        e = w.exec
        self.WS(w, i.args[0], int(self.V(w, i.args[1])[(e & -e).bit_length() - 1 if e else 0]), 1)

    def op_v_writelane_b32(self, w, i):
        lanes = np.zeros(LANES, dtype=bool)
        lanes[self.S(w, i.args[2], 1) & 63] = True
        w.vset(i.args[0], np.full(LANES, self.S(w, i.args[1], 1), dtype=U32), lanes)

    def op_v_permlane32_swap_b32_e32(self, w, i):
        d, s = i.args[0], i.args[1]
        a, b = self.V(w, d), self.V(w, s)
        na, nb = a.copy(), b.copy()
        na[32:], nb[:32] = b[:32], a[32:]
        every = np.ones(LANES, dtype=bool)
        w.vset(d, na, every)
        w.vset(s, nb, every)
    op_v_permlane32_swap_b32 = op_v_permlane32_swap_b32_e32

    def op_v_accvgpr_write_b32(self, w, i): self.WV(w, i.args[0], self.V(w, i.args[1]))
    def op_v_accvgpr_read_b32(self, w, i): self.WV(w, i.args[0], self.V(w, i.args[1]))
    def op_v_accvgpr_mov_b32(self, w, i): self.WV(w, i.args[0], self.V(w, i.args[1]))

    # ------------------------------------------------ MFMA (lane layouts: _MFMA_LAYOUT)
    def _halves(self, w, o, fp16):
        arr = w.v if o.kind == "v" else w.a
        w.check_read(o.kind, o.idx, 4)
        regs = arr[o.idx:o.idx + 4]
        h = np.empty((LANES, 8), dtype=np.uint32)
        for r in range(4):
            h[:, 2 * r] = regs[r] & 0xFFFF
            h[:, 2 * r + 1] = regs[r] >> 16
        if fp16:
            return h.astype(np.uint16).view(np.float16).astype(np.float64)
        return bf16_to_f32(h).astype(np.float64)

    def _mfma(self, w, i, m, fp16):
        dst, A, B, C = i.args
        nacc = 16 if m == 32 else 4
        k = 256 // m * 2  # 16 for 32x32, 32 for 16x16
        a, b = self._halves(w, A, fp16), self._halves(w, B, fp16)
        rows, ks, drow, dcol = _MFMA_LAYOUT[m]
        Am = np.zeros((m, k))
        Bm = np.zeros((k, m))
        Am[rows, ks] = a.reshape(-1)
        Bm[ks, rows] = b.reshape(-1)
        out = (Am @ Bm)[drow, dcol]
        if C.kind in ("v", "a"):
            arr = w.v if C.kind == "v" else w.a
            w.check_read(C.kind, C.idx, nacc)
            c = f32(arr[C.idx:C.idx + nacc]).astype(np.float64)
        else:
            c = np.full((nacc, LANES), float(C.val))
        res = u32((out + c).astype(np.float32))
        arr = w.v if dst.kind == "v" else w.a
        for r in range(nacc):
            w.check_write(dst.kind, dst.idx + r)
            arr[dst.idx + r] = res[r]

    def op_v_mfma_f32_32x32x16_bf16(self, w, i): self._mfma(w, i, 32, False)
    def op_v_mfma_f32_32x32x16_f16(self, w, i): self._mfma(w, i, 32, True)
    def op_v_mfma_f32_16x16x32_bf16(self, w, i): self._mfma(w, i, 16, False)
    def op_v_mfma_f32_16x16x32_f16(self, w, i): self._mfma(w, i, 16, True)

    # ------------------------------------------------ global memory
    def _gaddr(self, w, i, vaddr, saddr):
        if saddr is None or saddr.kind == "off":
            a = w.vget64(vaddr)
        else:
            a = U64(self.S(w, saddr, 2)) + self.V(w, vaddr).astype(U64)
        off = i.mods.get("offset", 0)
        return a + U64(off) if off >= 0 else a - U64(-off)

    def _queue_load(self, w, queue, dst, vals, lanes, extra=None):
        op = {"smem": False, "writes": [], **(extra or {})}
        for r in range(vals.shape[0]):
            key = (dst.kind, dst.idx + r)
            prior = w.pend.get(key)
            if prior is not None and not any(prior is o for o in queue):
                raise Hazard(f"load into {key[0]}{key[1]} while a load of the other counter into it is outstanding")
            op["writes"].append((key, vals[r].copy(), lanes.copy()))
        queue.append(op)
        for key, _, _ in op["writes"]:
            w.pend[key] = op
        return op

    def _gload(self, w, i, nbytes):
        dst, vaddr = i.args[0], i.args[1]
        addr = self._gaddr(w, i, vaddr, i.args[2] if len(i.args) > 2 else None)
        lanes = w.active()
        vals = np.zeros((max(nbytes // 4, 1), LANES), dtype=U32)
        for l in np.nonzero(lanes)[0]:
            raw = self.m.mem.read(int(addr[l]), nbytes)
            if nbytes >= 4:
                vals[:, l] = raw.view(np.uint32)
            else:  # ushort / ubyte: zero-extended
                vals[0, l] = int.from_bytes(raw.tobytes(), "little")
        self._queue_load(w, w.vm, dst, vals, lanes)

    def op_global_load_dword(self, w, i): self._gload(w, i, 4)
    def op_global_load_dwordx2(self, w, i): self._gload(w, i, 8)
    def op_global_load_dwordx3(self, w, i): self._gload(w, i, 12)
    def op_global_load_dwordx4(self, w, i): self._gload(w, i, 16)
    def op_global_load_ushort(self, w, i): self._gload(w, i, 2)
    def op_global_load_ubyte(self, w, i): self._gload(w, i, 1)

    def _gstore(self, w, i, nbytes):
        vaddr, data = i.args[0], i.args[1]
        addr = self._gaddr(w, i, vaddr, i.args[2] if len(i.args) > 2 else None)
        n = max(nbytes // 4, 1)
        w.check_read(data.kind, data.idx, n)
        regs = (w.v if data.kind == "v" else w.a)[data.idx:data.idx + n]
        for l in np.nonzero(w.active())[0]:
            self.m.mem.write(int(addr[l]), np.frombuffer(regs[:, l].astype(np.uint32).tobytes()[:nbytes], np.uint8))
        w.vm.append({"smem": False, "writes": []})

    def op_global_store_dword(self, w, i): self._gstore(w, i, 4)
    def op_global_store_dwordx2(self, w, i): self._gstore(w, i, 8)
    def op_global_store_dwordx3(self, w, i): self._gstore(w, i, 12)
    def op_global_store_dwordx4(self, w, i): self._gstore(w, i, 16)
    def op_global_store_short(self, w, i): self._gstore(w, i, 2)
    def op_global_store_byte(self, w, i): self._gstore(w, i, 1)

    def op_global_load_lds_dwordx4(self, w, i):
        """16 bytes per active lane from global memory to LDS at M0 + offset + 16 * lane; the
        bytes land when a vmcnt wait retires the copy."""
        addr = self._gaddr(w, i, i.args[0], i.args[1] if len(i.args) > 1 else None)
        base = (w.m0 & 0x3FFFF) + i.mods.get("offset", 0)
        copies, span = [], []
        for l in np.nonzero(w.active())[0]:
            raw = self.m.mem.read(int(addr[l]), 16).copy()
            la = base + 16 * int(l)
            self.m.lds_check(w, la, 16)
            if la + 16 > LDS_COPY_LIMIT:
                raise Fault(f"LDS copy to {la:#x}: the library keeps its copies below {LDS_COPY_LIMIT:#x}")
            copies.append((la, raw))
            span.append((la, 16, True))
        op = {"smem": False, "writes": [], "lds_copy": copies, "lds_span": span}
        for la, _ in copies:
            w.wg.copying[la:la + 16] = w.wid + 1
            w.wg.touch(w.wid, la, 16, True)
        w.vm.append(op)
        w.wg.lds_ops[w.wid].append(op)

    # ------------------------------------------------ scratch
    def _paddr(self, w, i, vaddr, saddr):
        a = np.zeros(LANES, dtype=np.int64)
        if vaddr.kind != "off":
            a += self.V(w, vaddr).astype(np.int64)
        if saddr.kind != "off":
            a += self.S(w, saddr, 1)
        return a + i.mods.get("offset", 0)

    def _scratch_load(self, w, i, n):
        dst, vaddr, saddr = i.args
        a = self._paddr(w, i, vaddr, saddr)
        lanes = w.active()
        size = w.priv.shape[1]
        vals = np.zeros((n, LANES), dtype=U32)
        for l in np.nonzero(lanes)[0]:
            ad = int(a[l])
            if ad < 0 or ad + 4 * n > size:
                raise Fault(f"scratch read {ad}+{4 * n} beyond the {size}-byte private segment")
            vals[:, l] = w.priv[l, ad:ad + 4 * n].view(np.uint32)
            if not w.priv_written[l, ad:ad + 4 * n].all():
                self.m.note_once(("scratch", i.line), f"line {i.line}: scratch read of bytes never written "
                                 f"({i.text})")
        self._queue_load(w, w.vm, dst, vals, lanes)

    def _scratch_store(self, w, i, n):
        vaddr, data, saddr = i.args
        a = self._paddr(w, i, vaddr, saddr)
        w.check_read(data.kind, data.idx, n)
        regs = (w.v if data.kind == "v" else w.a)[data.idx:data.idx + n]
        size = w.priv.shape[1]
        for l in np.nonzero(w.active())[0]:
            ad = int(a[l])
            if ad < 0 or ad + 4 * n > size:
                raise Fault(f"scratch write {ad}+{4 * n} beyond the {size}-byte private segment")
            w.priv[l, ad:ad + 4 * n] = np.frombuffer(regs[:, l].astype(np.uint32).tobytes(), np.uint8)
            w.priv_written[l, ad:ad + 4 * n] = True
        w.vm.append({"smem": False, "writes": []})

    def op_scratch_load_dword(self, w, i): self._scratch_load(w, i, 1)
    def op_scratch_load_dwordx2(self, w, i): self._scratch_load(w, i, 2)
    def op_scratch_load_dwordx3(self, w, i): self._scratch_load(w, i, 3)
    def op_scratch_load_dwordx4(self, w, i): self._scratch_load(w, i, 4)
    def op_scratch_store_dword(self, w, i): self._scratch_store(w, i, 1)
    def op_scratch_store_dwordx2(self, w, i): self._scratch_store(w, i, 2)
    def op_scratch_store_dwordx3(self, w, i): self._scratch_store(w, i, 3)
    def op_scratch_store_dwordx4(self, w, i): self._scratch_store(w, i, 4)

    # ------------------------------------------------ LDS
    def _lds_read(self, w, i, parts, nreg, transpose=False):
        """``parts``: per active lane, a list of (address, bytes) read in order."""
        lanes = w.active()
        vals = np.zeros((nreg, LANES), dtype=U32)
        span = []
        for l in np.nonzero(lanes)[0]:
            chunks = []
            for la, n in parts(l):
                self.m.lds_check(w, la, n)
                w.wg.touch(w.wid, la, n, False)
                span.append((la, n, False))
                chunks.append(w.wg.lds[la:la + n])
            vals[:, l] = np.concatenate(chunks).view(np.uint32)
        if transpose:
            # 16-lane groups: lane j holds row j (4 halfwords) of a 16x4 matrix M; lane i
            # receives M[i/4][i%4], M[4 + i/4][i%4], M[8 + i/4][i%4], M[12 + i/4][i%4]
            h = np.stack([vals[0] & 0xFFFF, vals[0] >> 16, vals[1] & 0xFFFF, vals[1] >> 16], axis=1)
            out = np.zeros_like(h)
            for g in range(4):
                blk = h[16 * g:16 * g + 16]
                for li in range(16):
                    out[16 * g + li] = [blk[4 * e + li // 4, li % 4] for e in range(4)]
            vals = np.stack([out[:, 0] | (out[:, 1] << 16), out[:, 2] | (out[:, 3] << 16)])
        op = self._queue_load(w, w.lgkm, i.args[0], vals, lanes, {"lds_span": span})
        w.wg.lds_ops[w.wid].append(op)

    def _base(self, w, i):
        """Per-lane LDS address operand: the second operand of a read, the first of a write."""
        return self.V(w, i.args[1] if i.op.startswith("ds_read") else i.args[0]).astype(np.int64)

    def _ds_read(self, w, i, n, transpose=False):
        a = self._base(w, i) + i.mods.get("offset", 0)
        self._lds_read(w, i, lambda l: [(int(a[l]), n)], n // 4, transpose)

    def _ds_read2(self, w, i, size, stride):
        a = self._base(w, i)
        o0, o1 = i.mods.get("offset0", 0) * size * stride, i.mods.get("offset1", 0) * size * stride
        self._lds_read(w, i, lambda l: [(int(a[l]) + o0, size), (int(a[l]) + o1, size)], 2 * size // 4)

    def op_ds_read_b32(self, w, i): self._ds_read(w, i, 4)
    def op_ds_read_b64(self, w, i): self._ds_read(w, i, 8)
    def op_ds_read_b128(self, w, i): self._ds_read(w, i, 16)
    def op_ds_read_b64_tr_b16(self, w, i): self._ds_read(w, i, 8, transpose=True)
    def op_ds_read2_b32(self, w, i): self._ds_read2(w, i, 4, 1)
    def op_ds_read2_b64(self, w, i): self._ds_read2(w, i, 8, 1)
    def op_ds_read2st64_b32(self, w, i): self._ds_read2(w, i, 4, 64)

    def _lds_write(self, w, i, parts):
        """``parts``: per active lane, a list of (address, uint8 data)."""
        span = []
        for l in np.nonzero(w.active())[0]:
            for la, data in parts(l):
                self.m.lds_check(w, la, len(data))
                w.wg.touch(w.wid, la, len(data), True)
                w.wg.lds[la:la + len(data)] = data
                span.append((la, len(data), True))
        op = {"smem": False, "writes": [], "lds_span": span}
        w.lgkm.append(op)
        w.wg.lds_ops[w.wid].append(op)

    def _reg_bytes(self, w, o, n, nbytes):
        w.check_read(o.kind, o.idx, n)
        regs = (w.v if o.kind == "v" else w.a)[o.idx:o.idx + n]
        return lambda l: np.frombuffer(regs[:, l].astype(np.uint32).tobytes()[:nbytes], np.uint8)

    def _ds_write(self, w, i, nbytes):
        a = self._base(w, i) + i.mods.get("offset", 0)
        data = self._reg_bytes(w, i.args[1], max(nbytes // 4, 1), nbytes)
        self._lds_write(w, i, lambda l: [(int(a[l]), data(l))])

    def _ds_write2(self, w, i, stride):
        a = self._base(w, i)
        o0, o1 = i.mods.get("offset0", 0) * 4 * stride, i.mods.get("offset1", 0) * 4 * stride
        d0, d1 = self._reg_bytes(w, i.args[1], 1, 4), self._reg_bytes(w, i.args[2], 1, 4)
        self._lds_write(w, i, lambda l: [(int(a[l]) + o0, d0(l)), (int(a[l]) + o1, d1(l))])


    def op_ds_write_b8(self, w, i): self._ds_write(w, i, 1)
    def op_ds_write_b16(self, w, i): self._ds_write(w, i, 2)
    def op_ds_write_b32(self, w, i): self._ds_write(w, i, 4)
    def op_ds_write_b64(self, w, i): self._ds_write(w, i, 8)
    def op_ds_write_b128(self, w, i): self._ds_write(w, i, 16)
    def op_ds_write2_b32(self, w, i): self._ds_write2(w, i, 1)
    def op_ds_write2st64_b32(self, w, i): self._ds_write2(w, i, 64)

    def op_ds_bpermute_b32(self, w, i):
        dst, vaddr, data = i.args
        src = ((self.V(w, vaddr).astype(np.int64) + i.mods.get("offset", 0)) >> 2) & 63
        d = self.V(w, data)
        lanes = w.active()
        vals = np.where(lanes[src], d[src], 0).astype(U32)[None, :]
        self._queue_load(w, w.lgkm, dst, vals, lanes)


def _install_compares():
    ops = {"eq": np.equal, "ne": np.not_equal, "lt": np.less, "le": np.less_equal,
           "gt": np.greater, "ge": np.greater_equal}
    for nm, f in ops.items():
        for kind in ("u32", "i32", "u64", "i64", "f32"):
            for enc in ("e32", "e64"):
                setattr(Semantics, f"op_v_cmp_{nm}_{kind}_{enc}",
                        lambda self, w, i, f=f, kind=kind: self._vcmp(w, i, f, kind))
        setattr(Semantics, f"op_v_cmp_{nm}_u16_sdwa", lambda self, w, i, f=f: self._vcmp(w, i, f, "u16"))
    unordered = {"nlt": lambda a, b: ~(a < b), "ngt": lambda a, b: ~(a > b), "nge": lambda a, b: ~(a >= b),
                 "nle": lambda a, b: ~(a <= b), "neq": lambda a, b: ~(a == b),
                 "lg": lambda a, b: (a < b) | (a > b), "u": lambda a, b: np.isnan(a) | np.isnan(b),
                 "o": lambda a, b: ~(np.isnan(a) | np.isnan(b))}
    for nm, f in unordered.items():
        for enc in ("e32", "e64"):
            setattr(Semantics, f"op_v_cmp_{nm}_f32_{enc}", lambda self, w, i, f=f: self._vcmp(w, i, f, "f32"))
    scmp = {"eq": lambda a, b: a == b, "lg": lambda a, b: a != b, "gt": lambda a, b: a > b,
            "ge": lambda a, b: a >= b, "lt": lambda a, b: a < b, "le": lambda a, b: a <= b}
    for nm, f in scmp.items():
        for ty in ("u32", "i32"):
            setattr(Semantics, f"op_s_cmp_{nm}_{ty}", lambda self, w, i, f=f, ty=ty: self._scmp(w, i, f, ty == "i32"))

            def k(self, w, i, f=f, ty=ty):
                a, c = self.S(w, i.args[0], 1), i.args[1].val & 0xFFFF
                if ty == "i32":
                    a, c = _sx32(a), _sx16(c)
                w.scc = int(f(a, c))
            setattr(Semantics, f"op_s_cmpk_{nm}_{ty}", k)
    for nm in ("eq", "lg"):
        setattr(Semantics, f"op_s_cmp_{nm}_u64", lambda self, w, i, f=scmp[nm]: self._scmp(w, i, f, False, 2))


_install_compares()


# ---------------------------------------------------------------- machine
class Machine:
    """One kernel: its instructions, the memory it sees, and the checks of a replay."""

    def __init__(self, asm_path, func, mem, kernarg_addr, lds_bytes, block, priv_bytes=0):
        self.instrs, self.labels = parse_function(asm_path, func)
        self.mem, self.kernarg = mem, kernarg_addr
        self.lds_bytes, self.block, self.priv_bytes = max(lds_bytes, 4), block, priv_bytes
        self.notes, self._seen = [], set()
        self.steps = 0
        self.executed = [0] * len(self.instrs)  # wave-level executions of each instruction
        sem = Semantics(self)
        self.handlers = [getattr(sem, "op_" + ins.op, None) for ins in self.instrs]
        self.missing = sorted({ins.op for ins, h in zip(self.instrs, self.handlers) if h is None})

    def op_counts(self):
        """Wave-level executions per mnemonic over the work groups run so far: what the
        SQ_INSTS_* counters count per dispatch, for the groups replayed."""
        out = {}
        for ins, n in zip(self.instrs, self.executed):
            if n:
                out[ins.op] = out.get(ins.op, 0) + n
        return out

    def note_once(self, key, msg):
        if key not in self._seen:
            self._seen.add(key)
            self.notes.append(msg)

    def run_group(self, wg_id, sgprs, max_steps=50_000_000):
        """Runs one work group.  ``sgprs`` are the system SGPRs after the kernarg pointer
        (the work-group ids the kernel descriptor enables)."""
        if self.missing:
            raise NotImplementedError(f"no semantics for {self.missing}")
        nw = (self.block + 63) // 64
        wg = WorkGroup(self, wg_id, nw)
        for w in wg.waves:
            w.s[0], w.s[1] = self.kernarg & M32, self.kernarg >> 32
            for k, x in enumerate(sgprs):
                w.s[2 + k] = x
            w.v[0] = np.arange(64 * w.wid, 64 * w.wid + 64, dtype=np.uint32)
            if self.block - 64 * w.wid < 64:
                w.exec = (1 << (self.block - 64 * w.wid)) - 1
        start = self.steps
        executed = self.executed
        while True:
            for w in wg.waves:
                while not w.done and not w.at_barrier:
                    ins = self.instrs[w.pc]
                    executed[w.pc] += 1
                    w.pc += 1
                    try:
                        self.handlers[w.pc - 1](w, ins)
                    except (Fault, Hazard) as e:
                        raise type(e)(f"work group {wg_id} wave {w.wid}, line {ins.line} ({ins.text}): {e}") from None
                    self.steps += 1
                    if self.steps - start > max_steps:
                        raise Hazard(f"work group {wg_id}: more than {max_steps} steps")
            live = [w for w in wg.waves if not w.done]
            if not live:
                break
            if not all(w.at_barrier for w in live):
                raise Hazard(f"work group {wg_id}: no wave can proceed")
            wg.end_interval()
            for w in live:
                w.at_barrier = False
        wg.end_interval()
        return wg

    # ---- completion of memory ops
    def retire(self, w, counter, keep):
        queue = w.vm if counter == "vm" else w.lgkm
        while len(queue) > keep:
            op = queue.pop(0)
            for key, vals, lanes in op["writes"]:
                if w.pend.get(key) is op:
                    del w.pend[key]
                kind, idx = key
                if kind == "s":
                    w.s[idx] = vals
                else:
                    (w.v if kind == "v" else w.a)[idx][lanes] = vals[lanes]
            for la, data in op.get("lds_copy", ()):
                w.wg.lds[la:la + len(data)] = data
                w.wg.copying[la:la + len(data)] = 0
            if "lds_span" in op:
                ops = w.wg.lds_ops[w.wid]
                for k, o in enumerate(ops):
                    if o is op:
                        del ops[k]
                        break

    def lds_check(self, w, addr, n):
        if addr < 0 or addr + n > self.lds_bytes:
            raise Fault(f"LDS access {addr}+{n} beyond the {self.lds_bytes}-byte allocation")
        own = w.wg.copying[addr:addr + n]
        if own.any():
            raise Hazard(f"LDS bytes {addr}+{n} accessed while a copy of wave {int(own[own != 0][0]) - 1} "
                         "into them is outstanding")
