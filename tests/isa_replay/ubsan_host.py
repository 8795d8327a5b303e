"""The library's host code under UndefinedBehaviorSanitizer, driven with boundary arguments.

``build()`` compiles every ``csrc/*.hip`` host-only with ``-fsanitize=undefined`` (host side
only; no device code is built) and links it with the launch recorder of ``host.py`` into
``_build/ubsan/libtattn_ubsan.so``: a copy of the library whose kernel launches are
recorded instead of run.  ``python -m isa_replay.ubsan_host <seed> <calls>`` (from ``tests/``)
calls every entry point with argument sets built from valid calls in which one to three
arguments take boundary values (0, 1, tile edges, 2^16, 2^24, 2^31 - 1, negatives, huge
strides, misaligned or NULL pointers, bad flags).  UBSan aborts the process on the first
undefined operation (signed overflow, bad shift, invalid conversion, ...).  For every call
the library accepts, each recorded launch must have a legal shape: grid x in [1, 2^31 - 1],
grid y and z in [1, 65535], 1 to 1024 threads a group.  It prints one JSON line with, per
entry point, the calls made, accepted and rejected.

Pointers are fake device addresses; the library never reads device memory on the host,
and the recorder never runs a kernel, so nothing here dereferences them.
"""
from __future__ import annotations

import ctypes
import glob
import json
import os
import random
import subprocess
import sys

from . import host as H

UB = os.path.join(H.BUILD, "ubsan")


def _runtime_dir():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.ubsan_standalone-x86_64.so")
    if not hits:
        raise FileNotFoundError("clang's UBSan runtime (libclang_rt.ubsan_standalone-x86_64.so) not found")
    return os.path.dirname(hits[0])


def build():
    """Returns the path of the UBSan host library; rebuilds what is stale."""
    import concurrent.futures as cf
    B = H._pkg_build()
    H.build(asm_sources=())  # the launch recorder
    os.makedirs(UB, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
    headers = sorted(glob.glob(os.path.join(B.CSRC, "*.h"))) + [os.path.join(B.ROOT, "include", "tiled_attn.h")]
    flags = [f for f in B.COMMON if f != "-O3"] + ["-O1", "-g", "--offload-host-only",
                                                    "-Xarch_host", "-fsanitize=undefined",
                                                    "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs, jobs = [], []
    for src in srcs:
        out = os.path.join(UB, os.path.basename(src)[:-4] + ".o")
        objs.append(out)
        if H._stale(out, [src, *headers]):
            jobs.append([B._hipcc(), *flags, "-c", src, "-o", out])
    with cf.ThreadPoolExecutor(max_workers=min(8, max(1, len(jobs)))) as ex:
        list(ex.map(H._run, jobs))
    lib = os.path.join(UB, "libtattn_ubsan.so")
    rec = os.path.join(H.BUILD, "liblaunch_record.so")
    if H._stale(lib, [*objs, rec]):
        need = set()
        for o in objs:
            nm = subprocess.run(["nm", "-u", o], capture_output=True, text=True).stdout
            need |= {w for w in nm.split() if w.startswith("__hip_fatbin_")}
        stubs = os.path.join(UB, "fatbin_symbols.c")
        with open(stubs, "w") as fh:
            for s in sorted(need):
                fh.write(f"const unsigned char {s}[16] __attribute__((weak));\n")
        stub_o = os.path.join(UB, "fatbin_symbols.o")
        H._run(["gcc", "-c", "-fPIC", "-x", "c", stubs, "-o", stub_o])
        rt = _runtime_dir()
        H._run(["g++", "-shared", "-fPIC", "-o", lib, *objs, stub_o, "-L" + H.BUILD, "-llaunch_record",
                "-Wl,-rpath," + H.BUILD, "-L" + rt, "-lclang_rt.ubsan_standalone-x86_64", "-Wl,-rpath," + rt])
    return lib


# ---------------------------------------------------------------- the driver
INT_MAX, INT_MIN = 2**31 - 1, -2**31
SIZES = [0, 1, 2, 7, 15, 16, 17, 63, 64, 65, 127, 128, 129, 4095, 4096, 65535, 65536, 65537,
         2**20, 2**24 - 1, 2**24, 2**24 + 1, 2**30, INT_MAX, -1, -7, INT_MIN]
STRIDES = [0, 8, 64, 128, 2**20, 2**24 - 8, 2**24, 2**31 - 8, 2**31, 2**40, 2**62, -8, -2**31, 3, 4]
GOOD = 0x7F0000000000   # fake device addresses, 256-byte aligned
MISALIGNED = GOOD + 8


def _strides(*v):
    return (ctypes.c_int64 * 3)(*v)


class Driver:
    def __init__(self, lib_path, seed):
        self.rec = ctypes.CDLL(os.path.join(H.BUILD, "liblaunch_record.so"), mode=ctypes.RTLD_GLOBAL)
        self.rec.record_get.restype = ctypes.POINTER(H._Launch)
        from tiled_attention_attn_amd import _lib as L
        self.L = L
        self.lib = L.declare_signatures(ctypes.CDLL(lib_path))
        self.rng = random.Random(seed)
        self.stats = {}
        self.keep = []
        self.k = 1.0

    # ---- helpers
    def pick(self, good, bad, p=0.25):
        return self.rng.choice(bad) if self.rng.random() < p * self.k else good

    def ptr(self, p=0.06):
        r = self.rng.random()
        p *= self.k
        return None if r < p else (MISALIGNED if r < 2 * p else GOOD)

    def size(self, good, p=0.2):
        return self.pick(good, SIZES, p)

    def strides(self, N, H_, D):
        good = [H_ * N * D, N * D, D]
        if self.rng.random() < 0.3 * self.k:
            good[self.rng.randrange(3)] = self.rng.choice(STRIDES)
        s = _strides(*good)
        self.keep.append(s)
        return s

    def mask(self):
        L, r = self.L, self.rng
        if r.random() < 0.15:
            return None
        flags = r.choice([0, 1, 2, 4, 8, 3, 5, 6, 9, 15, 16, 1 << 16, 1 | (7 << 16), 0xFFFFFFFF])
        d = L.attn_mask_desc(flags=flags, window_left=r.choice([-1, 0, 1, 512, 2048, INT_MAX, INT_MIN]),
                             window_right=r.choice([-1, 0, 1, 512, INT_MAX]),
                             block_size=r.choice([0, 1, 16, 128, -1, INT_MAX]),
                             doc_offsets=r.choice([None, GOOD, MISALIGNED]),
                             num_docs=r.choice([0, 1, 3, 65536, INT_MAX, -1]),
                             doc_stride=r.choice([0, 2, 4, 65537, INT_MAX, -1]))
        self.keep.append(d)
        return ctypes.byref(d)

    def smod(self):
        L, r = self.L, self.rng
        if r.random() < 0.6:
            return None
        d = L.attn_score_mod(flags=r.choice([0, 1, 2, 4, 8, 5, 12, 3, 16, 0xFFFFFFFF]),
                             slopes=r.choice([None, GOOD]), rel_bias=r.choice([None, GOOD]),
                             rel_radius=r.choice([0, 1, 32, 1023, 1024, INT_MAX, -1]),
                             softcap=r.choice([30.0, 0.0, -1.0, float("inf"), float("nan"), 1e-30]))
        self.keep.append(d)
        return ctypes.byref(d)

    def blockmask(self, B, Hq, Nq, Nk):
        r = self.rng
        nq, nk = (max(Nq, 0) + 127) // 128, (max(Nk, 0) + 127) // 128
        bm = self.L.attn_blockmask(Bm=self.pick(r.choice([1, max(B, 1)]), SIZES, 0.15),
                                   Hm=self.pick(r.choice([1, max(Hq, 1)]), SIZES, 0.15),
                                   nQt=self.pick(nq, SIZES, 0.15), nKt=self.pick(nk, SIZES, 0.15),
                                   part_num=self.ptr(0.03), part_idx=self.ptr(0.03),
                                   full_num=self.ptr(0.03), full_idx=self.ptr(0.03))
        self.keep.append(bm)
        return bm

    def shape(self):
        r = self.rng
        if r.random() < 0.1:
            # valid but huge head and batch counts: products of sizes past 2^31 (decode-shaped
            # rows, so attn_fwd_auto may take split-KV)
            Hkv = r.choice([1, 256, 65535])
            return (r.choice([32767, 32768, 65535]), Hkv * r.choice([1, 1, 2]) if Hkv < 65535 else Hkv,
                    Hkv, r.choice([1, 16]), r.choice([512, 4096]), r.choice([64, 128]))
        D = self.pick(r.choice([64, 128]), [0, 32, 96, 256, -64])
        Hkv = self.size(r.choice([1, 2, 8]), 0.1)
        G = r.choice([1, 2, 4, 8])
        Hq = self.size(Hkv * G if Hkv > 0 else 1, 0.1)
        B = self.size(r.choice([1, 2, 16]), 0.15)
        Nq = self.size(r.choice([1, 16, 300, 4096, 32768]), 0.2)
        Nk = self.size(r.choice([Nq, 512, 32768, 1]), 0.2)
        return B, Hq, Hkv, Nq, Nk, D

    def dtype(self):
        return self.pick(self.rng.choice([0, 1]), [2, -1, 7], 0.1)

    def scale(self):
        return self.pick(0.125, [0.0, -1.0, float("inf"), float("nan"), 1e-38, 3e38], 0.1)

    def check_launches(self, name):
        n = self.rec.record_count()
        for i in range(n):
            l = self.rec.record_get(i).contents
            g, b = l.grid, l.block
            ok = (1 <= g.x <= INT_MAX and 1 <= g.y <= 65535 and 1 <= g.z <= 65535 and
                  1 <= b.x <= 1024 and b.y == 1 and b.z == 1)
            if not ok:
                raise AssertionError(f"{name}: launch {i} has grid ({g.x}, {g.y}, {g.z}) block "
                                     f"({b.x}, {b.y}, {b.z})")
        self.rec.record_clear()
        return n

    def call(self, name, *args):
        st = getattr(self.lib, name)(*args)
        s = self.stats.setdefault(name, {"calls": 0, "accepted": 0, "launches": 0})
        s["calls"] += 1
        n = self.check_launches(name)
        if st == 0:
            s["accepted"] += 1
            s["launches"] += n
        elif n:
            raise AssertionError(f"{name} returned {st} after recording {n} launches")
        return st

    # ---- entry points
    def fwd(self, which):
        B, Hq, Hkv, Nq, Nk, D = self.shape()
        args = [self.ptr(), self.strides(Nq, Hq, D), self.ptr(), self.strides(Nk, Hkv, D),
                self.ptr(), self.strides(Nk, Hkv, D), self.ptr(), self.strides(Nq, Hq, D),
                self.pick(GOOD, [None, MISALIGNED], 0.1), B, Hq, Hkv, Nq, Nk, D, self.dtype(), self.scale(),
                self.mask(), self.smod()]
        if which == "attn_fwd":
            self.call(which, *args, None)
        elif which == "attn_fwd_blockmask":
            self.call(which, *args, ctypes.byref(self.blockmask(B, Hq, Nq, Nk)), None)
        else:
            ws = self.pick(1 << 62, [0, 16, 1 << 20], 0.3)
            self.call(which, *args, self.ptr(0.05), ws, None)
            plan = self.L.attn_auto_plan()
            self.call("attn_fwd_auto_plan", B, Hq, Hkv, Nq, Nk, D, args[-1], ctypes.byref(plan))

    def decode(self, which):
        r = self.rng
        B, Hq, Hkv, Lq, Nk, D = self.shape()
        ps = self.pick(r.choice([16, 1, 64]), [0, -16, 3, 65536, INT_MAX], 0.15)
        max_pages = self.size((max(Nk, 1) + max(ps, 1) - 1) // max(ps, 1), 0.15)
        S = self.pick(r.choice([1, 4, 9]), [0, -1, 65536, 65537, INT_MAX], 0.15)
        pool = self.pick(40000, [0, 1, -1, 2**31, 2**40], 0.1)
        bt_stride = self.pick(max(max_pages, 0), [0, -1, 2**31, 2**40], 0.1)
        q_st = self.strides(Lq, Hq, D)
        head = [self.ptr(), q_st, self.ptr(), self.ptr(), pool, self.ptr(), bt_stride, self.ptr(),
                max_pages, B, Hq, Hkv, Lq, D, self.dtype(), ps, S, self.scale(), self.mask(), self.smod()]
        if which == "attn_decode_splitkv":
            self.call(which, *head, self.ptr(0.05), self.ptr(0.05), None)
            self.call("attn_decode_combine", self.ptr(0.05), self.ptr(0.05), B, Hq, Lq, S, D, self.dtype(),
                      self.ptr(), self.strides(Lq, Hq, D), self.ptr(0.3), None)
            for fn, a in (("attn_decode_ws_o_bytes", (B, Hq, Lq, D, S)), ("attn_decode_ws_lse_bytes", (B, Hq, Lq, S)),
                          ("attn_decode_num_splits", (B, Hkv, max_pages, self.pick(256, [0, -1, INT_MAX], 0.2)))):
                getattr(self.lib, fn)(*a)
        else:
            self.call(which, *head, self.ptr(), self.strides(Lq, Hq, D), self.ptr(0.3), None)

    def bwd(self, which):
        B, Hq, Hkv, Nq, Nk, D = self.shape()
        sq, sk = self.strides(Nq, Hq, D), self.strides(Nk, Hkv, D)
        args = [self.ptr(), sq, self.ptr(), sk, self.ptr(), sk, self.ptr(), sq, self.ptr(), sq,
                self.ptr(), self.ptr(), sq, self.ptr(), sk, self.ptr(), sk, B, Hq, Hkv, Nq, Nk, D,
                self.dtype(), self.scale(), self.mask(), self.smod()]
        self.lib.attn_bwd_workspace_bytes(B, Hq, Nq)
        ws_bytes = self.pick(1 << 40, [0, 4, 1 << 20], 0.2)
        if which == "attn_bwd":
            self.call(which, *args, self.ptr(0.05), ws_bytes, None)
        else:
            bm = self.blockmask(B, Hq, Nq, Nk)
            bt = self.L.attn_blockmask(Bm=bm.Bm, Hm=bm.Hm, nQt=self.pick(bm.nKt, SIZES, 0.1),
                                       nKt=self.pick(bm.nQt, SIZES, 0.1), part_num=self.ptr(0.03),
                                       part_idx=self.ptr(0.03), full_num=self.ptr(0.03), full_idx=self.ptr(0.03))
            self.keep.append(bt)
            self.call(which, *args, ctypes.byref(bm), ctypes.byref(bt), self.ptr(0.05), ws_bytes, None)
            self.call("attn_blockmask_transpose", ctypes.byref(bm), ctypes.byref(bt), self.ptr(0.05),
                      self.pick(1 << 40, [0, 1], 0.2), None)

    def build_blockmask(self):
        B, Hq, Hkv, Nq, Nk, D = self.shape()
        bm = self.blockmask(B, Hq, Nq, Nk)
        self.lib.attn_blockmask_bytes(bm.Bm, bm.Hm, bm.nQt, bm.nKt)
        self.call("attn_build_blockmask", self.mask(), self.ptr(0.5), B, Nq, Nk, ctypes.byref(bm), None)

    def run(self, n):
        ops = [lambda: self.fwd("attn_fwd"), lambda: self.fwd("attn_fwd_blockmask"),
               lambda: self.fwd("attn_fwd_auto"), lambda: self.decode("attn_decode_splitkv"),
               lambda: self.decode("attn_decode_noalloc"), lambda: self.bwd("attn_bwd"),
               lambda: self.bwd("attn_bwd_blockmask"), self.build_blockmask]
        for i in range(n):
            # how often arguments leave their valid values: none (only the drawn sizes vary,
            # so more calls are accepted and launch), some, or the full rates
            self.k = self.rng.choice([0.0, 0.3, 1.0])
            ops[i % len(ops)]()
            if len(self.keep) > 4096:
                self.keep = self.keep[-64:]
        for c in range(-20, 1):
            self.lib.attn_status_str(c)
        return self.stats


def main(argv):
    seed, n = int(argv[0]), int(argv[1])
    lib = argv[2] if len(argv) > 2 else os.path.join(UB, "libtattn_ubsan.so")
    stats = Driver(lib, seed).run(n)
    print(json.dumps(stats, sort_keys=True), flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
