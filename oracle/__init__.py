"""Plain fp64 CPU oracle for partial-context patch attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library (no kernels,
headers, planners or helpers); the only thing both sides consume is the seeded
synthetic input generator, which holds none of the method's arithmetic.

Sources (web pages, cited by title and section):

* "Partially Conditioned Patch Parallelism for Accelerated Diffusion Model
  Inference" (pith.science review page) -- sections "What carries the
  argument" and "Core claim": each patch attends to its own activation plus
  the nearest p-fraction (of the neighbour's height) of each adjacent patch,
  taken from the previous step's (stale) activations; the partial rows are
  concatenated into the local key and value sets.  Minor comment on Sec. 3.3:
  the attention is multi-head scaled dot-product attention.
* "ScaleDiff: Higher-Resolution Image Synthesis via Efficient and
  Model-Agnostic Diffusion" (atlas.scime.ai summary) -- section "Approach":
  the query tiles partition the token map, and the keys/values of a tile are
  its own rectangle grown by a halo on every side and clipped at the map
  border, so neighbouring tiles share keys (Neighborhood Patch Attention);
  the same section adds a guidance step that pulls the latent's low
  frequencies towards a reference.

Modules:
  attention -- membership predicates, tier-0 (per-pair loops) and tier-1
               (per-tile dense fp64) attention, useful-pair counts.
  guidance  -- Gaussian low-pass (reflect-101) and the structure-guidance blend.
"""
