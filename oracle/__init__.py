"""Plain, slow, obviously-correct CPU oracle for layer-streamed NF4-LoRA training.

THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The GPU path (the C-ABI library and its Python binding) never
imports, calls or links anything here, and nothing here imports the GPU path:
the two share no code, tables or constants.

Modules
-------
``oracle.nf4``    blockwise NF4 codebook / quantize / dequantize
``oracle.model``  decoder-layer forward/backward with LoRA, LM head, SFT/DPO
                  losses and one SGD step, in numpy (dtype follows the inputs:
                  float64 for parity and finite differences, float32 for the
                  timed CPU baseline)

Sources.  The method is described on five web pages about the "Soup" CLI:
  * "Soup: Fine-Tune an 8B Model on a 4 GB GPU" (lucaberton.com), section
    "The Core Idea: Layer Streaming": the frozen weights live off the GPU (host
    memory or a disk) and reach it layer by layer, through a copy stream of
    their own, when a pass needs them; they may be stored as NF4; the LoRA
    adapter is the only trained state; DPO's reference model is that same
    base run without the adapter.
  * "Show HN: Fine-tune an 8B model on a 4 GB laptop GPU" (elseif.net),
    first and second paragraphs: policy and reference log-probabilities from
    two runs of the same base, bit-exact against a non-streamed run.
  * axbrief.com article, section "Beyond Memory: The Layer Streaming
    Breakthrough": streaming is bit-exact with respect to resident execution.
Because the method is exact, the oracle computes the plain *resident*
definition of one training step; streaming is only a schedule.

The pages print no formulas.  Where they are silent the oracle takes the
plainest reading (listed in each function's docstring):  NF4 = 16-level
normal-quantile code with exact zero and per-64-element absmax scale; LoRA
y = x W + s (x A) B; Llama/Qwen-style decoder layer (RMSNorm, rotate-half
RoPE, causal GQA attention, SwiGLU MLP, no biases); DPO loss
-log sigmoid(beta((pc - rc) - (pr - rr))).

Parity status.  Every function has a pin in tests/test_oracle_*.py (closed
forms, invariants, brute force, finite differences).  Whole-stack values at
the large (3B-/8B-shaped) sizes are "parity unpinned" beyond those component
pins: no printed values exist for them.
"""
