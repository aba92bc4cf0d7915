"""MI355X-native fused row softmax.

The compute path is a hand-written HIP library for gfx950 behind a C ABI
(``include/row_wise_softmax.h``); this package holds that library's sources,
its ctypes binding and the seeded input generators.  PyTorch is used only for
device memory and streams.
"""
from .binding import (  # noqa: F401
    attention,
    attention_fwd,
    softmax,
    softmax_fwd,
    softmax_fwd_split,
    softmax_fwd_causal,
    softmax_fwd_kernel,
    softmax_select,
    kernel_table,
    library_path,
    SoftmaxError,
)
