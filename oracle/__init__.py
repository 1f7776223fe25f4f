"""CPU oracle for spectral transform coding of the KV cache.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, fp64 statement of
what the codec computes. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or run it; the product path (the HIP library and its
Python binding) never does, and shares no code, tables or helpers with it.

Sources (cited by page title and section; the pages are web summaries of the
papers):

* "Sintesi Tecnica: SPECTRA" (gist.science, Italian summary of SPECTRA),
  sections "Metodologia: SPECTRA" (observations 1-3) and "La Pipeline di
  SPECTRA" (steps 1-3): second-moment basis, reverse water-filling, 0-bit
  channels dropped, per-token quantization appended to a latent cache,
  on-the-fly reconstruction for attention.
* SPECTRA abstract (arxivdaily.com, English abstract): the cache is re-read in
  full at every generated token; rotation into the cache's own statistics.
* "Technisch Overzicht: Ablatie, Statistische Inferentie en Validatie voor
  KV-Cache Compressie" (gist.science, Dutch summary), sections "Experimentele
  Opstelling" (TurboQuant: randomized Walsh-Hadamard rotation plus a
  data-independent Beta Lloyd-Max codebook; SpectralQuant: per-head
  eigenbasis calibrated on representative tokens with water-filling bits;
  relMSE metric) and "Belangrijkste Bijdragen" (Plain-KV without rotation,
  SQU-KV uniform allocation).

Where the pages leave a step open, the reading taken is stated at the function
that implements it. Parity status of every function is listed in the module
docstrings: each is pinned by a test in tests/test_oracle_*.py against closed
forms, textbook routines, brute force or published tables, except where a
docstring says "parity unpinned".
"""
from . import codec, rht  # noqa: F401
