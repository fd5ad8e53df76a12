"""Helpers of the GPU parity tests: device checks and numpy <-> torch moves."""
import sys

import numpy as np
import pytest
import torch


def require_gpu():
    """Skip when there is no GPU; fail when there is one but the HIP library
    is missing (the product has no CPU fallback)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delayed_scaling_amd as ds
    ds.lib()
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name
    return ds


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits):
    """numpy uint16 bf16 bit patterns -> contiguous bf16 CUDA tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_u8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda()


def bf16_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_bits(x):
    return int(np.float32(x).view(np.uint32))
