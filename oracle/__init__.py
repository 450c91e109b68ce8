"""CPU oracle for one rank's share of a fully sharded (ZeRO-3 / FSDP FULL_SHARD) training step.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain reference that the GPU library is
checked against. Only the test suite, the smoke check of the graft entry point and the CPU-baseline
leg of the benchmark may import it. The GPU product path never imports, calls or falls back to it,
and it shares no code with that path (no kernels, headers, helpers, constants or table
generators); it imports nothing from the GPU package either.

What it computes, and where each piece comes from (page titles as published):

* layout      -- flatten a unit's tensors into one 1-D vector and give rank k the contiguous slice
                 floor(kP/N) .. floor((k+1)P/N)-1.  "FSDP: Fully Sharded Data Parallel Training at
                 Scale", passage on sharding a linear layer.
* bf16        -- bfloat16 keeps fp32's 8-bit exponent and a 7-bit mantissa; conversion from fp32
                 is IEEE round-to-nearest-even on the bit pattern.  Same page, mixed-precision
                 passage.
* step        -- reduce the F bf16 gradient contributions of the slice in fp32 (the arithmetic a
                 reduce-scatter performs: the sum, kept only for the owner's slice; the fp32 reduce
                 dtype of the mixed-precision passage), then the Adam update of the fp32 master,
                 first and second moment shards (the moments are exponential moving averages of the
                 gradient and of its square, kept in fp32: memory-breakdown passage), then the bf16
                 copy of the updated master written into the flat layout that the next all-gather
                 serves (communication-pattern passage).
* accounting  -- the 16-bytes-per-parameter state accounting (2 + 2 + 4 + 8 for mixed precision).
* clip        -- the global gradient norm of a sharded gradient and the clip coefficient (same
                 page, gradient-clipping passage).
* step also holds the fp32 gradient-shard accumulation across micro-batches and the step that
  consumes such an fp32 shard (mixed-precision passage).
* reshard     -- shards of one world size (and padding multiple) turned into another's (same page,
                 checkpointing passage: local state dicts are tied to one configuration).

Precision: the pages fix the precision of every stored quantity on this path (fp32 master, m, v
and reduction; bf16 params and gradients), so the oracle computes in float32 with one IEEE
rounding per operation and no fused multiply-add, in a fixed operation order.  A float64 shadow of
the same recurrence (``step.adamw_update_f64``) exists only as a diagnostic.
"""

from . import accounting, bf16, clip, layout, reshard, step  # noqa: F401
