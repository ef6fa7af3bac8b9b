"""MI355X (gfx950) batch-1 MoE + FP8 LM-head decode path.

The compute path lives in the HIP library libwsx.so (built from csrc/); the
Python modules here only marshal arguments (`ops`), describe workloads
(`configs`) and draw seeded synthetic inputs (`inputs`).  Importing `ops`
loads the library and raises if it has not been built.
"""

__all__ = ["configs", "inputs"]
