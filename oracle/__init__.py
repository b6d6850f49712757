"""CPU fp64 oracle for the tensor-parallel Transformer block and the
vocab-sharded cross-entropy.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it. It shares no code with the HIP path.

Every step is the plain definition, written out in float64 NumPy, one step
after another in the order the pages give them, so that it can be read
against the pages by eye:

* ``block``  -- LayerNorm, QKV, per-head softmax attention, output
  projection, residuals, GELU/SwiGLU MLP, and the backward pass of all of it,
  evaluated as R tensor-parallel shards whose partial sums are added at the
  two reduction points (R = 1 is the unsharded block);
* ``xent``   -- cross-entropy over vocab-sharded logits, following the
  three-reduction scheme (global max, target logit, sum of exponentials);
* ``embed``  -- the vocab-parallel input embedding: masked lookup per shard,
  summed over shards, and its adjoint (scatter-add into the shard's rows);
* ``lmhead`` -- the vocab-parallel output layer feeding ``xent``: logits slice
  z_r = h W_r^T per shard, and the gradients dW_r and sum_r dz_r W_r;
* ``dropout`` -- counter-based dropout masks (Philox4x32-10 from its published
  definition) with the tensor-parallel seed scheme, used by ``block``.

Pages cited (short key -> page):

* [Lab06]     "LLM Lab notes 06: assembling a Megatron-style Transformer
  Block from scratch" (chat.ai-hpc.org, guide/11-training/
  llm-lab-06-megatron-block); sections 1-5, listing steps (1)-(8).
* [TP-block]  "02 - How the whole Transformer block is sharded"
  (llm-infra-atlas.github.io, parallel/02_tp_sp/02_transformer_block);
  sections 1 MLP, 2 Attention, 3 vocab-parallel embedding,
  4 vocab-parallel cross entropy, 5 TP RNG.
* [MLM-notes] "Megatron-LM" notes (huajishe.fun); headings
  ColumnParallelLinear, RowParallelLinear, in-layer sharding, load balance.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (finite differences, shard-sum identities, closed
forms, brute force on tiny inputs, an independent float64 autograd
cross-check). No function is "parity unpinned".
"""
from . import block, embed, lmhead, xent  # noqa: F401
