"""MI355X-native DLRM embedding-bag + pairwise-interaction hot path.

The compute lives in a HIP shared library (libdlrm_embbag.so, C ABI declared in
include/dlrm_embbag.h); `sparse_embedding_lookup_dlrm_amd.ops` is a thin ctypes
binding over it. Importing this package loads nothing; the library is opened on
first use and an ImportError/RuntimeError is raised if it is missing.
"""
__all__ = ["synth"]
