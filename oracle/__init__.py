"""CPU oracle (test infrastructure only).

Plain, slow, float64 reference implementations written from the ReSET pages:
``nvfp4_oracle`` (formats, quantization, GEMV), ``reset_oracle`` (entropy
and the step-aware temperature rule) and ``sampler_oracle`` (top-p sampling
at the chosen temperature).  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this package; the HIP library shares nothing with it.
"""
