"""Plain CPU oracle for layer-streamed LoRA fine-tuning (TEST INFRASTRUCTURE ONLY).

This package is the slow, obviously-correct reference that the HIP path is checked
against.  It is NOT part of the product: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import or call
it.  It shares no code, tables or constants with the HIP library; both sides only
consume the same seeded inputs.

Sources (the pages this method is described on):

* "Soup: Fine-Tuning an 8B Model on a 4 GB Laptop GPU, One Layer at a Time"
  (toknow.ai), opening paragraphs: frozen base in CPU RAM, copied one layer at a
  time, double-buffered; 4-bit base; forward bit-exact against a resident run.
* the lachieslifestyle.com how-to on fine-tuning Llama 3.1 8B on a 4 GB GPU with
  Soup (16 Aug 2026), section "What Soup layer streaming changes": two-buffer VRAM
  pool, layer re-read during
  backward recomputation; section "Step 5: Enable 4-bit layer streaming": the
  ``lora: r 16, alpha 32, target_modules: auto`` and ``stream_buffers: 2`` knobs.
* "Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU" (codeinktechnologies.com),
  sections "Quantization: Shrink the Weights" (NF4, nested quantisation) and
  "LoRA and QLoRA: Train a Fraction of the Parameters" (frozen base, trainable
  low-rank adapters in full precision), "Gradient Checkpointing and Paged
  Optimizers" (recompute in backward).
* "Soup CLI fine-tunes Llama-3.1-8B on a 4 GB laptop GPU ..." (thetesserapress.com),
  second and third paragraphs: dedicated copy stream, peak bounded by one layer,
  DPO reference = same streamed base with adapters off.

Where the pages are silent the module docstrings state the reading taken.

Modules
-------
nf4     NF4 codebook, blockwise quantisation, nibble packing, double quantisation,
        dequantisation (encoding steps; every function pinned by tests).
model   LoRA projection and the Llama-style decoder layer, forward and hand-derived
        backward, in float64.
stack   the layer stack (forward with checkpoints, recompute backward), the
        adapters-off reference pass, and a simulated two-slot streaming pool.
optim   the AdamW update of the adapters (decoupled, lr-scaled weight decay).
head    the output head (final RMSNorm, logits), SFT cross entropy and the DPO
        objective with hand-derived logit gradients, and the head backward.
adapters  adapter file names (PEFT convention), the safetensors container, the
        integrity record (per-tensor CRC-32) and a checker of a file against a stack.
"""
