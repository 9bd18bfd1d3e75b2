"""MI355X-native tree-packed chunkwise KDA: host planner, gfx950 HIP kernels
and a thin ctypes binding over the C-ABI library (libkda_tree.so).

The library is loaded lazily by tree_packed_chunkwise_amd.binding; importing
this package does not touch the GPU.
"""
__all__ = ["binding", "synth"]
