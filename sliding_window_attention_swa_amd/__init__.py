"""Sliding-window attention over a two-pool paged KV cache, MI355X (gfx950).

The product is the C-ABI library libswa.so (include/swa.h) built from csrc/;
`swa` is its thin ctypes binding (importing it loads the library and fails if
it is missing), `workloads` the seeded synthetic inputs, `build` the hipcc
build.  Submodules are imported explicitly; importing the package itself loads
nothing.
"""

__all__ = ["swa", "workloads", "build"]
