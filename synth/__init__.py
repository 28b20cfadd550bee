"""Seeded synthetic inputs for the GrowPage boundary engine.

This package only *constructs inputs* (page pools, page tables, summaries, decode
queries, RoPE tables).  It computes none of the engine's outputs, and it is the only
code shared by the CPU oracle (``oracle/``) and the HIP path's tests and bench.
"""
