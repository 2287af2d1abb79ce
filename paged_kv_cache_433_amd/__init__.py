"""MI355X (gfx950) paged KV-cache decode: HIP kernels behind a C ABI."""
