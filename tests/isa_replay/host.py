"""Builds what a replay needs and runs recorded launches on the emulator.

``build`` compiles, into ``tests/isa_replay/_build``:
  * the gfx950 assembly of chosen kernel sources, with the library's own flags;
  * every source host-only, linked with ``launch_record.c`` into a copy of the library
    whose kernel launches are recorded instead of run.
``Replay`` calls that copy through the C ABI with host buffers standing in for device
memory, then runs each recorded launch work group by work group.
"""
from __future__ import annotations

import ctypes
import glob
import os
import re
import subprocess

import numpy as np
import yaml

from . import emulator as E

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(HERE, "_build")


def _pkg_build():
    from tiled_attention_attn_amd import build as B  # the library's compiler flags and paths
    return B


def _stale(out, deps):
    return not os.path.exists(out) or any(os.path.getmtime(d) > os.path.getmtime(out) for d in deps)


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)} failed:\n{r.stderr[-4000:]}")


def build(asm_sources=("bwd",)):
    """Returns (host library path, {source: assembly path}); rebuilds what is stale."""
    import concurrent.futures as cf
    B = _pkg_build()
    hipcc = B._hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
    headers = sorted(glob.glob(os.path.join(B.CSRC, "*.h"))) + [os.path.join(B.ROOT, "include", "tiled_attn.h")]
    jobs = []
    asm = {}
    for name in asm_sources:
        src = os.path.join(B.CSRC, name + ".hip")
        out = os.path.join(BUILD, name + ".s")
        asm[name] = out
        if _stale(out, [src, *headers]):
            jobs.append([hipcc, *B.COMMON, "--offload-device-only", "-S", src, "-o", out])
    objs = []
    for src in srcs:
        out = os.path.join(BUILD, os.path.basename(src)[:-4] + ".host.o")
        objs.append(out)
        if _stale(out, [src, *headers]):
            jobs.append([hipcc, *B.COMMON, "--offload-host-only", "-c", src, "-o", out])
    with cf.ThreadPoolExecutor(max_workers=min(8, max(1, len(jobs)))) as ex:
        list(ex.map(_run, jobs))
    rec_src = os.path.join(HERE, "launch_record.c")
    rec = os.path.join(BUILD, "liblaunch_record.so")
    if _stale(rec, [rec_src, *objs]):
        # a host-only object still names the device image of its source; define those symbols
        need = set()
        for o in objs:
            nm = subprocess.run(["nm", "-u", o], capture_output=True, text=True).stdout
            need |= set(re.findall(r"__hip_fatbin_[0-9a-f]+", nm))
        stubs = os.path.join(BUILD, "fatbin_symbols.c")
        with open(stubs, "w") as fh:
            for s in sorted(need):
                fh.write(f"const unsigned char {s}[16] __attribute__((weak));\n")
        _run(["gcc", "-O1", "-fPIC", "-shared", "-o", rec, rec_src, stubs, "-ldl"])
    lib = os.path.join(BUILD, "libtattn_host.so")
    if _stale(lib, [*objs, rec]):
        _run(["g++", "-shared", "-fPIC", "-o", lib, *objs, "-L" + BUILD, "-llaunch_record",
              "-Wl,-rpath," + BUILD])
    return lib, asm


# ---------------------------------------------------------------- kernel metadata
class Kernels:
    """Kernel descriptors (.amdhsa_*) and argument metadata of assembly files."""

    def __init__(self, paths):
        self.where, self.desc, self.meta = {}, {}, {}
        for p in paths:
            txt = open(p).read()
            for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", txt, re.S):
                d = {}
                for ln in m.group(2).split("\n"):
                    t = ln.split()
                    if len(t) == 2 and t[0].startswith(".amdhsa_"):
                        d[t[0][8:]] = int(t[1], 0)
                self.desc[m.group(1)] = d
                self.where[m.group(1)] = p
            mm = re.search(r"\.amdgpu_metadata\n(.*?)\.end_amdgpu_metadata", txt, re.S)
            if mm:
                body = "\n".join(l for l in mm.group(1).split("\n") if l.strip() and not l.startswith("\t"))
                for k in yaml.safe_load(body)["amdhsa.kernels"]:
                    self.meta[k[".name"]] = k

    def explicit_args(self, name):
        return [a for a in self.meta[name][".args"] if a[".value_kind"] in ("by_value", "global_buffer")]

    def kernarg(self, name, launch):
        """The kernel argument segment of a launch: its recorded arguments plus the hidden
        grid and group sizes."""
        md = self.meta[name]
        buf = np.zeros(md[".kernarg_segment_size"] + 64, dtype=np.uint8)
        explicit = self.explicit_args(name)
        for a in md[".args"]:
            off, sz, kind = a[".offset"], a[".size"], a[".value_kind"]
            if kind in ("by_value", "global_buffer"):
                if len(explicit) == 1:
                    raw = launch["arg0"][:sz]
                else:
                    if sz > 8:
                        raise NotImplementedError("a multi-argument kernel with an argument over 8 bytes")
                    raw = launch["argv"][explicit.index(a)][:sz]
                buf[off:off + sz] = np.frombuffer(raw, dtype=np.uint8)
            elif kind.startswith("hidden_block_count_"):
                buf[off:off + 4] = np.frombuffer(np.uint32(launch["grid"]["xyz".index(kind[-1])]).tobytes(), np.uint8)
            elif kind.startswith("hidden_group_size_"):
                buf[off:off + 2] = np.frombuffer(np.uint16(launch["block"]["xyz".index(kind[-1])]).tobytes(), np.uint8)
            elif kind == "hidden_grid_dims":
                g = launch["grid"]
                buf[off:off + 2] = np.frombuffer(np.uint16(3 if g[2] > 1 else (2 if g[1] > 1 else 1)).tobytes(), np.uint8)
        return buf


class _Dim3(ctypes.Structure):
    _fields_ = [("x", ctypes.c_uint32), ("y", ctypes.c_uint32), ("z", ctypes.c_uint32)]


class _Launch(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 512), ("grid", _Dim3), ("block", _Dim3), ("shmem", ctypes.c_size_t),
                ("arg0", ctypes.c_uint8 * 2048), ("argv", (ctypes.c_uint8 * 8) * 32), ("nargs", ctypes.c_int),
                ("handle", ctypes.c_void_p)]


# ---------------------------------------------------------------- replay
class Replay:
    """A host-only library copy whose launches are recorded, host buffers registered as
    device memory, and the emulator to run the recorded launches."""

    def __init__(self, asm_sources=("bwd",)):
        lib_path, asm = build(asm_sources)
        self.rec = ctypes.CDLL(os.path.join(BUILD, "liblaunch_record.so"), mode=ctypes.RTLD_GLOBAL)
        self.rec.record_get.restype = ctypes.POINTER(_Launch)
        self.rec.record_symbol_memory.restype = ctypes.c_void_p
        self.rec.record_symbol_bytes.restype = ctypes.c_size_t
        assert self.rec.record_struct_size() == ctypes.sizeof(_Launch)
        from tiled_attention_attn_amd import _lib
        self.lib = _lib.declare_signatures(ctypes.CDLL(lib_path))
        self.kernels = Kernels(list(asm.values()))
        for name in self.kernels.meta:
            n = len(self.kernels.explicit_args(name))
            if n > 1:
                self.rec.record_set_nargs(name.encode(), n)
        self._names = self._internal_names(lib_path)
        self.mem = E.Memory()
        self.mem.add(self.rec.record_symbol_memory(),
                     np.ctypeslib.as_array((ctypes.c_uint8 * self.rec.record_symbol_bytes()).from_address(
                         self.rec.record_symbol_memory())), "static device array")
        self.keep = []
        self.notes = []
        self.ran = []

    def _internal_names(self, lib_path):
        """Kernel handles without a dynamic symbol (anonymous namespaces): from the full symbol table."""
        out = subprocess.run(["nm", lib_path], capture_output=True, text=True).stdout
        syms = {}
        for ln in out.split("\n"):
            t = ln.split()
            if len(t) == 3:
                syms.setdefault(t[2], int(t[0], 16))
        base = ctypes.cast(self.lib.attn_abi_version, ctypes.c_void_p).value - syms["attn_abi_version"]
        return {base + off: nm for nm, off in syms.items() if "kernel" in nm and "__device_stub__" not in nm}

    def register(self, **tensors):
        """Makes CPU tensors visible to replayed kernels at their own addresses."""
        for name, t in tensors.items():
            if t is None:
                continue
            n = max(t.untyped_storage().nbytes(), 1)
            addr = t.untyped_storage().data_ptr()
            self.mem.add(addr, np.ctypeslib.as_array((ctypes.c_uint8 * n).from_address(addr)), name)
            self.keep.append(t)

    def recorded(self):
        out = []
        for i in range(self.rec.record_count()):
            l = self.rec.record_get(i).contents
            name = l.name.decode() or self._names.get(l.handle, "")
            out.append(dict(name=name, grid=(l.grid.x, l.grid.y, l.grid.z), block=(l.block.x, l.block.y, l.block.z),
                            shmem=l.shmem, arg0=bytes(l.arg0), argv=[bytes(l.argv[k]) for k in range(32)]))
        self.rec.record_clear()
        return out

    def run(self, only=None, groups=None):
        """Runs the launches recorded since the last call (those whose name contains one of
        ``only``, if given; ``groups(launch)`` may pick work-group indices)."""
        for L in self.recorded():
            if only and not any(s in L["name"] for s in only):
                continue
            self.run_launch(L, groups(L) if groups else None)

    def run_launch(self, L, group_ids=None):
        name = L["name"]
        if name not in self.kernels.desc:
            raise KeyError(f"no assembly for launched kernel {name!r}")
        d = self.kernels.desc[name]
        if d["user_sgpr_count"] != 2 or L["block"][1:] != (1, 1):
            raise NotImplementedError(f"{name}: kernarg-pointer-only user SGPRs and 1-D blocks are replayed")
        ka = self.mem.alloc(self.kernels.kernarg(name, L).tobytes(), "kernarg " + name)
        m = E.Machine(self.kernels.where[name], name, self.mem, ka, d.get("group_segment_fixed_size", 0) + L["shmem"],
                      L["block"][0], d.get("private_segment_fixed_size", 0))
        gx, gy, gz = L["grid"]
        ids = [(x, y, z) for z in range(gz) for y in range(gy) for x in range(gx)]
        if group_ids is not None:
            ids = [ids[k] for k in group_ids]
        for t in ids:
            sg = [t[k] for k, axis in enumerate("xyz") if d.get(f"system_sgpr_workgroup_id_{axis}", int(axis == "x"))]
            m.run_group(t, sg)
        self.notes += [f"{name}: {n}" for n in m.notes]
        self.ran.append((name, L["grid"], m.steps))
        return m
