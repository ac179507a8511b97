"""MI355X-native discrete-diffusion denoising step (DiffusionGemma-style MoE LM).

Submodules: `configs` (shapes and workloads), `synth` (seeded synthetic
inputs), `dg` (binding of the C-ABI library libdg, built from `csrc/`),
`build` (hipcc build of libdg for gfx950).  Nothing is imported eagerly so
that the shape and input modules load without the library.
"""
