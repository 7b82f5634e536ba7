"""MI355X-native sparse-KV decode path of SpeContext (speculative context sparsity).

The compute path is the HIP library ``libspc.so`` (C-ABI, see include/spc.h);
``api`` is its thin ctypes binding and ``driver`` orders one decode step on HIP
streams.  ``workload`` draws the seeded synthetic inputs.  Importing this
package loads nothing; the library is loaded on first use of ``api`` and the
load fails loudly if it has not been built.
"""
__all__ = ["api", "driver", "workload"]
