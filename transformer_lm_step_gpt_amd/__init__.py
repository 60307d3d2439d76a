"""GPT-2 training step on one MI355X (gfx950): HIP kernels behind a C ABI.

The binding (`transformer_lm_step_gpt_amd.gpt`) is imported lazily so that the
input generators can be used without a GPU or the built library.
"""

__all__ = ["inputs", "gpt"]
