"""Training-mode normalization forward/backward for AMD Instinct MI355X.

Submodules:
    normhip    -- the Python binding of the C ABI (include/normhip.h); loads
                  libnormhip.so and raises if it is not built
    workloads  -- seeded synthetic inputs (no normalization arithmetic)
    build      -- compiles libnormhip.so with hipcc for gfx950
"""
