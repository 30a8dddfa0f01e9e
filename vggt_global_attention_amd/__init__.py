"""MI355X-native VGGT Aggregator attention block (frame / global / register).

The compute lives in the HIP library libvggtattn.so (see include/libvggtattn.h);
`binding` is its ctypes binding and `api` a torch-tensor front end.  Submodules
are imported lazily so that the seeded input generator can be used without the
library.
"""

__all__ = ["api", "binding", "build", "configs", "synth"]
