"""fp64 CPU oracle for the Transformer-XL relative-attention step.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import anything here. The product (the HIP library and its
Python binding) never imports, calls or links this package, and this package
never imports the product: the two share no code. Inputs come from
``txl_synth`` (random draws only) or from values the pages print.

Every function is a plain, slow, literal reading of the pages, in float64:
explicit loops over queries, the mask rule evaluated per key, and the relative
embedding looked up by distance (no shift trick, no ring buffer, no tiling).

Pages cited (by title and section):
  [P1] zty624.github.io notes, "Transformer-XL" (sections "Segment-Level
       Recurrence", "Batched Tensor Contract", "Causal Mask With Memory",
       "Relative Positional Encoding", "Dimension Walkthrough", "Relative
       Shift Trick", "Relative Shift Golden Test", "Batched Streams", "Stream
       Sampler Contract", "Training Loop Sketch", ...)
  [P2] wq-win.github.io, "019 Transformer-XL" (section 3 pseudo-code and the
       worked example of a 4x12 score)
  [P3] iopencloud.com, "Transformer-XL与长序列建模" (section 2.2, the
       (q+u)/(q+v) form of the score)
  [P4] robocikowo.com, "Transformer-XL" (glossary: FIFO memory buffer,
       four-term score, sinusoidal relative embedding)

Parity status of each function (what pins it is listed in the tests):
  attention.allow, attention.rel_ids, attention.rel_attn   pinned
  attention.rel_attn_bwd                                   pinned (finite
      differences of rel_attn, torch fp64 autograd of a dense formulation,
      softmax identities)
  memory.tail_rows, tail, update_mems, update_rows        pinned
  stack.layer_norm, stack.gelu                             pinned (torch fp64)
  stack.sinusoid                                           parity unpinned
      (the pages only say "sinusoidal"; the formula is a stated reading,
       checked for internal properties only)
  stack.layer_forward (and its steps split_heads, merge_heads, context,
      r_for_memory, add_norm)                              pinned (closed
      forms: two torch fp64 LayerNorms with the sublayers off, torch fp64
      SDPA for the attention sublayer with u = v = W_R = 0, the pinned
      relative attention on raw states, the capacity-m table equal to the
      last m + L rows of the capacity-M one, head-permutation invariance;
      each pin fails on a planted mistake). The layer body itself (W^O,
      post-LayerNorm, GELU feed-forward) is a reading of this build: the
      pins fix how it is composed, not that the pages prescribe it.
  stack.segment_step_row, stack.stream                    pinned (the
      hand-unrolled recurrence; reset equals a fresh stream)
  stack.layer_backward, segment_backward_row,
      layer_norm_backward, gelu_grad                      pinned (central
      finite differences of the pinned forward for every entry of every
      weight, the segment input and the embedding rows, with the memory held
      fixed as the stop-gradient input it is; planted mistakes in the
      LayerNorm and GELU derivatives fail them)
  evaluation.row_streams                                   pinned (hand-worked
      example from the stream-state contract, stream invariants)
  evaluation.segment_nll                                   pinned (closed form,
      torch fp64 cross entropy)
"""
from . import attention, evaluation, memory, stack  # noqa: F401
