"""CPU oracle for block-diffusion denoising: TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 numpy implementation of what the HIP library computes:
causal prefill into a KV cache, one bidirectional denoising pass over an
all-[MASK] canvas, the confidence-ranked commit, and the append of a finished
canvas.  Only the tests, the package's smoke check and the benchmark's CPU
baseline may import it; the product path never does.  It shares no code with
the HIP path; both read their inputs from the `synth` module.

Sources (the three pages the method is described on):
  * rahulsharmavishwakarma.github.io, "Diffusion LLMs: what changes when you stop
    generating one token at a time" -- section 2 (reverse process, bidirectional
    attention, several commits per pass), section 4.1 (block diffusion), section
    4.2 (256-token canvas, causal prefill, bidirectional denoising, finished
    canvases appended to the KV cache, up to 48 steps), section 5 (confidence
    threshold commits).
  * b4rtaz.github.io, "Diffusion LLMs are not a good fit for distributed
    inference" -- canvas paragraph (256-token canvas, up to 48 steps).
  * agentlenshq.com, "DiffusionGemma: 4x Faster Text Generation via Parallel
    Diffusion" -- "Bi-directional Attention" (every canvas token attends to all
    others), "Parallel Generation and Hardware Efficiency" (26B MoE).

Parity status per function is stated in each module header.
"""
