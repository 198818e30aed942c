"""MI355X-native GR00T flow-matching DiT action head.

The compute path lives in the HIP library ``libgr00t_head.so`` (C-ABI declared
in include/gr00t_head.h); ``flow_matching_dit_amd.head`` is a thin ctypes
binding over it. Importing this package loads nothing; the library is opened on
first use and a missing library is an error, never a fallback.
"""
__all__ = ["synth"]
