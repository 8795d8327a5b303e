"""CPU replay of the library's compiled gfx950 kernels (test infrastructure).

``emulator`` runs the assembly that hipcc writes for a kernel (``-S``), wave by
wave and lane by lane, and checks every memory access and a few hazards of the
compiled code.  ``host`` builds that assembly and a host-only copy of the
library whose kernel launches are recorded instead of run, so a replay uses
exactly the launch arguments the library computes.
"""
