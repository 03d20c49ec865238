"""libmuon: the Muon optimizer step (momentum orthogonalised by quintic
Newton–Schulz) as hand-written HIP for MI355X (gfx950), behind a C ABI.

`binding` is the ctypes layer over libmuon.so (include/libmuon.h);
`build` compiles the library in-tree with hipcc.
"""

__all__ = ["binding", "build"]
