"""Seeded synthetic inputs for the hybrid compressed sparse attention hot path.

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only draws numbers and lays bytes out in memory: it holds none of
the method's arithmetic (no compression, scoring, selection or attention).

Modules:
  configs  -- the five workload shapes (tiny CSA, CSA decode, HCA decode,
              CSA prefill chunk, 1M-context CSA decode with fp8 KV)
  layout   -- paged cache byte layouts (bf16 rows, fp8_ds records, MXFP4 keys)
  gen      -- seeded generators producing logical tensors and paged buffers
"""
