"""long_context_swa_amd: causal sliding-window attention over a dual-pool KV cache on MI355X.

``long_context_swa_amd.swa``   the binding of the native library (include/swa.h); importing it
                               fails if ``lib/libswa.so`` has not been built.
``long_context_swa_amd.build`` builds ``lib/libswa.so`` with hipcc for gfx950.
"""
