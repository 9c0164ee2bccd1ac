"""libloopspec for AMD Instinct MI355X: pipelined self-speculative decoding of looped
Transformers (LoopSpec), hot path in hand-written HIP kernels behind a C ABI.

Modules:
  _lib      - ctypes binding of include/loopspec.h (fails loudly if the library is not built)
  engine    - device memory (weights, depth-indexed KV caches, hidden states, workspace)
  decoder   - host branch scheduler (spawn / gate / verify / prune / re-root), generate()
  copyprop  - copy-suffix candidates with shallow screening
  build_lib - hipcc build of libloopspec.so for gfx950
"""

import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libloopspec.so")


def load():
    """Import the native binding (raises ImportError when libloopspec.so is missing)."""
    from . import _lib
    return _lib
