"""Host arrays to device tensors for the GPU tests.

The seeded generators hand out read-only arrays (they are cached and
shared), and torch.from_numpy warns on a read-only buffer; every helper here
copies the array first, so the tensor owns writable host memory for the
moment it takes to copy it to the GPU.
"""
import numpy as np
import torch


def _to_device(a, dtype):
    return torch.from_numpy(np.array(a, dtype=dtype, order="C", copy=True)).cuda()


def dev_bf16(a):
    """bf16 bit patterns (uint16 or int16) as an int16 device tensor."""
    return _to_device(np.asarray(a).view(np.int16), np.int16)


def dev_i32(a):
    return _to_device(a, np.int32)


def dev_u8(a):
    return _to_device(a, np.uint8)


def dev_f32(a):
    return _to_device(a, np.float32)
