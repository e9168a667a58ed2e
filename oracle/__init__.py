"""CPU fp64 oracle for head-aware sparse decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this
package: only the test suite, the smoke check and the CPU-baseline leg of
the benchmark may import or call it.  It is plain numpy in float64, written
step by step from the method descriptions on the pages:

  * "Resumen Técnico: Autonomía de Cabezales (Autonomy-of-Heads, AoH)"
    (gist.science, paper 2608.06849; also its French twin) -- the effective
    rank labeller (`aoh`).
  * "FASA: Frequency-aware Sparse Attention" (gist.science, paper
    2602.03152) -- token importance prediction over dominant frequency
    chunks, top-N_fac selection and focused attention (`fasa`).
  * "El enrutamiento compartido entre capas acelera la atención dispersa 7
    veces ..." (seventnews.com, on "CLSA: You Only Index Once") -- one index
    computed once and reused by every layer sharing the KV cache (`clsa`).

It shares no code with the HIP library: inputs come from the seeded
generator package `synth`, widened exactly to float64.
"""
from . import aoh, clsa, fasa  # noqa: F401
