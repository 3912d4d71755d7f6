"""MI355X-native training step of a GPT-style decoder with a hand-written backward pass.

The compute path is the HIP library libgpt.so (gfx950 kernels behind a C ABI, declared in
include/gpt.h); `gpt_lm_step_amd.binding` is a thin ctypes layer over it, loaded on first use.
`configs` and `inputs` are host-side helpers (layouts, presets, seeded synthetic inputs).
"""
from . import configs, inputs  # noqa: F401
