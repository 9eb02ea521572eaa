"""MI355X-native GDN (Gated DeltaNet) layer: HIP kernels behind a C-ABI library."""
