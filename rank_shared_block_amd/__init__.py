"""MI355X-native theta-bundle reconstructed linear (HIP kernels behind a C ABI)."""
