"""CPU oracle (TEST INFRASTRUCTURE ONLY): a plain NumPy float64 implementation
of the MoE layer forward.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import it; the GPU library never does."""
