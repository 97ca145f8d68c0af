"""MI355X-native STEPQuant packed-state decode step.

``stepq``  -- Python binding of the C-ABI library ``libstepq.so`` (HIP kernels for gfx950).
``synth``  -- seeded synthetic workloads.
``planning`` -- product-side offline planning (calls the library's host allocators).
"""
