"""MI355X-native forward pass of one DeepSeekMoE layer (HIP kernels for gfx950 behind a C ABI)."""
