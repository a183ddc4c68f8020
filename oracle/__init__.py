"""Plain, slow CPU oracle of the SPECTRA-style KV transform codec.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the benchmark's CPU
baseline may import this package.  The library in `spectral_transform_coding_amd` never
imports or calls it, and it shares no code with the library: it re-derives every step from
the pages in float64 NumPy (float32 NumPy where the codec fixes float32 arithmetic).

Sources (page title, then section):
  [SPECTRA]  "SPECTRA: Pushing the KV Cache Beyond the 2-Bit Cliff via Spectral Transform
             Coding" (technical summary; sections Problem statement, Methodology,
             SPECTRA pipeline stages 1-3, Core contributions).
  [ABLATION] "Ablation, Statistical Inference, and Validation for KV-Cache Compression"
             (Methodology, Experimental setup, Core contributions 2-3).
  [SPECTRAL-KV] "Spectral-KV: SVD-projection KV cache compression" forum thread
             (Technical principle: 1 spectral profiling, 2 projection, 3 latent quantization;
             Usage).

Every function is pinned by a `-m "not gpu"` test against closed forms, invariants, special
cases that reduce to library routines, hand-computed examples or brute force.  The
closed-form W_O correction of the pipeline's first stage has no formula on the pages; its
least-squares reading leaves the attention output unchanged, so the decode applies a
caller-supplied W_O' as given and no oracle function computes a correction.
"""
from . import transform, allocation, quant, layout, attention, calibrate  # noqa: F401
