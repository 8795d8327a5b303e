"""Dry run of GPU test functions on the CPU, through the compiled kernels.

``python -m isa_replay.dryrun <test module> <function>[[k]] ...`` (from ``tests/``; every
parametrization of the function, or only its k-th) imports a GPU test module with the package's Python binding intact, but:

  * the binding's library is the host-only copy whose kernel launches are recorded
    (``host.Replay``), and every tensor whose pointer the binding passes (data, BlockMask
    lists, document offsets, ALiBi slopes, bias tables) is registered with the emulator
    as device memory;
  * tensors live on the CPU (the module's ``DEV`` becomes "cpu", BlockMask buffers too);
  * ``torch.cuda.synchronize()`` runs the launches recorded so far on the emulator, work
    group by work group, with its bounds, race and lane-mask checks.

So a GPU test's own code -- shapes, binding calls, oracle comparisons -- runs end to end
against the kernels' gfx950 assembly, and must pass as it would on the GPU.  Meant for
small GPU test cases: the emulator runs about a million wave instructions a minute.
This process patches torch.cuda, so run it in a process of its own.
"""
from __future__ import annotations

import importlib
import sys


def main(argv):
    import torch
    torch.cuda.is_available = lambda: True  # the test module imports the binding
    from . import emulator as E
    from .host import Replay
    from tiled_attention_attn_amd import _lib as L

    rp = Replay(("fwd", "fwd_pp", "bwd", "blockmask", "decode", "decode_noalloc"))
    seen, seen_notes = set(), set()

    def reg(t):
        if t is not None and t.untyped_storage().data_ptr() not in seen:
            seen.add(t.untyped_storage().data_ptr())
            rp.register(**{f"tensor{len(seen)}": t})

    ptr, struct, init = L._ptr, L.BlockMask.struct, L.BlockMask.__init__

    def ptr_reg(t):
        reg(t)
        return ptr(t)

    def struct_reg(self):
        for t in (self.part_num, self.part_idx, self.full_num, self.full_idx):
            reg(t)
        return struct(self)

    def init_cpu(self, Bm, Hm, Nq, Nk, device="cuda"):
        init(self, Bm, Hm, Nq, Nk, device="cpu")

    # Scratch bytes start as 0x7F (3.4e38 as a float, 2^31 - 129 as an integer): a read of
    # a spill slot never written is noted, and if its value were used the results or the
    # addresses would show it.  Any other note fails the run.
    E.PRIV_FILL = 0x7F

    def synchronize(*_):
        rp.run()
        bad = [n for n in rp.notes if "scratch read of bytes never written" not in n]
        for n in rp.notes:
            if n not in bad and n not in seen_notes:
                seen_notes.add(n)
                print(f"note (scratch filled with 0x7F): {n}", flush=True)
        if bad:
            raise AssertionError(f"replay notes: {bad}")

    mask_desc, smod_desc = L.Mask.desc, L.ScoreMod.desc

    def mask_desc_reg(self):
        reg(self.doc_offsets)
        return mask_desc(self)

    def smod_desc_reg(self):
        reg(self.alibi_slopes)
        reg(self.rel_bias)
        return smod_desc(self)

    L._ptr, L.BlockMask.struct, L.BlockMask.__init__ = ptr_reg, struct_reg, init_cpu
    L.Mask.desc, L.ScoreMod.desc = mask_desc_reg, smod_desc_reg
    L._on_device = lambda *a: None
    L._stream = lambda s: None
    L._lib = rp.lib
    torch.cuda.synchronize = synchronize
    torch.cuda.empty_cache = lambda: None
    # tests that call the C ABI directly pass the current stream's handle: the null stream
    torch.cuda.current_stream = lambda *a: type("Stream", (), {"cuda_stream": 0})()
    # and their tensors: any tensor whose address is taken counts as device memory
    data_ptr = torch.Tensor.data_ptr

    def data_ptr_reg(t):
        if t.numel():
            reg(t)
        return data_ptr(t)

    torch.Tensor.data_ptr = data_ptr_reg

    import pytest
    mod = importlib.import_module(argv[0])
    _to_cpu()
    for spec in argv[1:]:
        name, _, sel = spec.partition("[")
        fn = getattr(mod, name)
        calls = _parameter_sets(fn)
        if sel:
            calls = [calls[int(sel.rstrip("]"))]]
        for label, kwargs in calls:
            try:
                fn(**kwargs)
                synchronize()
                print(f"dry run passed: {argv[0]}::{name}{label}", flush=True)
            except pytest.skip.Exception as e:
                print(f"dry run skipped: {argv[0]}::{name}{label} ({e})", flush=True)


def _to_cpu():
    """Every loaded test module (the target and the helpers it imported from other test
    files): DEV = "cpu", and "cuda" default arguments of its functions become "cpu"."""
    import types
    for name, m in list(sys.modules.items()):
        if not (name.startswith("test_") or name == "gpu_util") or m is None:
            continue
        if getattr(m, "DEV", None) == "cuda":
            m.DEV = "cpu"
        for f in vars(m).values():
            if isinstance(f, types.FunctionType) and f.__defaults__ and "cuda" in f.__defaults__:
                f.__defaults__ = tuple("cpu" if d == "cuda" else d for d in f.__defaults__)


def _parameter_sets(fn):
    """(label, keyword arguments) of every parametrization of a test function, in the
    order pytest would make them (the last decorator's argument varies fastest)."""
    import itertools
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    axes = []
    for m in reversed(marks):  # decorators apply bottom-up
        names = [n.strip() for n in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
        ids = m.kwargs.get("ids")
        vals = list(m.args[1])
        axes.append([(ids[i] if ids else str(i), dict(zip(names, v if len(names) > 1 else (v,))))
                     for i, v in enumerate(vals)])
    out = []
    for combo in itertools.product(*axes):
        kw = {}
        for _, d in combo:
            kw.update(d)
        out.append(("[" + "-".join(lbl for lbl, _ in combo) + "]" if combo else "", kw))
    return out or [("", {})]


if __name__ == "__main__":
    main(sys.argv[1:])
