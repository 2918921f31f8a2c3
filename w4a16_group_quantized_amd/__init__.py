"""MI355X (gfx950) routed-expert W4A16 group-32 MoE layer.

The compute path lives in the HIP library ``libmoe_w4a16.so`` (C ABI declared
in ``include/moe_w4a16.h``); :mod:`w4a16_group_quantized_amd.ops` is a thin
ctypes binding over it.  Importing this package loads nothing; the library is
opened on first use and a missing library raises an error.
"""

__all__ = ["ops", "inputs"]
