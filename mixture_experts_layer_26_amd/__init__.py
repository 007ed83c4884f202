"""DeepSeekMoE layer (forward, bias update and backward) for AMD MI355X (gfx950).

The compute path is the C ABI of ``include/moe.h`` (``libmoe.so``, hand-written HIP
kernels); ``abi`` binds it with ctypes and ``layer`` holds device buffers for a whole
step. PyTorch is used for device memory and streams only.
"""
from . import abi  # noqa: F401
