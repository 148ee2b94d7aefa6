"""CPU oracle for the hybrid compressed sparse attention hot path (fp64, NumPy).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything here. The product
path (``hybrid_compressed_sparse_amd``) never imports it, and this package
never imports the product path: the two share no code. Inputs come from
``synth`` (seeded generators and byte layouts only).

Every function is the plain definition of what the DeepSeek-V4 pages describe,
written out in float64 with NumPy library primitives (matmul, exp, sort):

  formats   -- exact decoders of the stored number formats (bf16, OCP e4m3,
               OCP e2m1, UE8M0, fp8_ds records, MXFP4 rows) and the reference
               rounding rules used to check stored outputs
  method    -- the KV compressor, Lightning-Indexer scores, top-k selection,
               the sliding-window + compressed row set, and sparse MQA attention
  pipeline  -- one step of the path for a ``synth`` scenario, query by query

Where the pages leave a step open, the reading taken is stated next to the
function.
"""
