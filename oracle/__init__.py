"""CPU oracle of one denoising step of a discrete-diffusion MoE language model.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
numpy statement of what the GPU path computes.  Only the test-suite, the
`smoke()` check and the benchmark's CPU-baseline leg may import it; the
product library never calls it, and it shares no code with the HIP path
(only the seeded input generators feed both).

Sources: the DiffusionGemma technical report as summarised on the arXiv
abstract page (66bd.net mirror), the laozijiushiniubi.cn article (sections
1-5: block diffusion over a 256-token canvas, multinomial noise, causal prefix
with bidirectional canvas attention, self-conditioning, MoE 128 experts top-8,
entropy-ranked locking, temperature anneal, adaptive stop), the gxsgwd.com news
item (bidirectional attention inside each 256-token block) and the
chatpaper.ai English abstract.  Readings taken where the pages are silent are
listed in each module's docstring.

Modules
  rng      Philox4x32-10 (SC'11 definition), uniform mapping, own fp32 ln, Gumbel
  model    forward pass: prefix prefill (causal), canvas step (bidirectional),
           one-token autoregressive decode against the cache
  sampler  entropy, Gumbel-max sample, lock / re-randomise / stop, block loop,
           the autoregressive next-token sample

Parity unpinned: the whole-step output against the real DiffusionGemma (no
trained weights or reference implementation are available); every function
here is pinned piecewise by tests/test_oracle_*.py.
"""
from . import rng, model, sampler  # noqa: F401
