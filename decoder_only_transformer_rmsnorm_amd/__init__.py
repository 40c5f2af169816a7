"""MI355X-native forward pass of a pre-norm decoder-only Transformer (RMSNorm, RoPE,
causal GQA attention, SwiGLU), built from hand-written HIP kernels behind a C ABI."""
