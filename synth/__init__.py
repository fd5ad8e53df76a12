"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds random-number recipes only: no quantization, scaling or GEMM
arithmetic.  Both the HIP path and the oracle receive the same host arrays
made here (or, for bf16_normal_device, the same device tensor's bits).

Recipe (the pages train on their own models and data, which are not
available, so every tensor is synthetic with the shapes of the pages'
workloads):
  * a bf16 tensor is torch.randn(shape) drawn from a CPU generator seeded with
    `seed`, multiplied by sigma in float32 and rounded to bf16 (nearest-even);
  * "outliers" multiplies a Bernoulli(0.01) subset, drawn from the same
    generator after the normal draw, by 50;
  * seeds follow 1000*config + 100*step + tensor id (X=1, W=2, G=3, bias=4,
    A=5, B=6) so every tensor of every workload is reproducible on its own.
"""
import numpy as np
import torch

TENSOR_ID = {"X": 1, "W": 2, "G": 3, "bias": 4, "A": 5, "B": 6}


def seed_for(config, step, tensor, layer=0):
    """Seed of one tensor of one workload step (layer adds 10000*layer)."""
    return 1000 * config + 100 * step + TENSOR_ID[tensor] + 10000 * layer


def bf16_normal(shape, seed, sigma=1.0, outliers=False):
    """bf16 bit patterns (numpy uint16) of sigma * N(0, 1), optionally with
    1% of the elements multiplied by 50."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32) * float(sigma)
    if outliers:
        mask = torch.rand(tuple(shape), generator=g) < 0.01
        x = torch.where(mask, x * 50.0, x)
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_normal_device(shape, seed, sigma=1.0, outliers=False, device="cuda"):
    """The bf16_normal recipe drawn on the GPU from a device generator seeded
    with `seed` (a different stream of numbers than bf16_normal's), as a bf16
    device tensor: for workloads too large to draw on the host at every step.
    Whoever checks a result against the oracle hands it this tensor's bits,
    copied to the host."""
    g = torch.Generator(device).manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32) * float(sigma)
    if outliers:
        mask = torch.rand(tuple(shape), generator=g, device=device) < 0.01
        x = torch.where(mask, x * 50.0, x)
    return x.to(torch.bfloat16)


def bf16_normal_sequence(shapes, seed, sigma=1.0):
    """Several bf16 tensors drawn one after another from one CPU generator
    seeded with `seed` (the tiny workload draws X, W and bias this way)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    out = []
    for shape in shapes:
        x = torch.randn(tuple(shape), generator=g, dtype=torch.float32) * float(sigma)
        out.append(x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    return out


def bf16_from_float(values):
    """bf16 bit patterns of given float values (nearest-even), for hand-made
    small inputs."""
    t = torch.as_tensor(np.asarray(values, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def random_codes(shape, seed, allowed=None):
    """Random 8-bit codes; `allowed` restricts them to a given set of codes."""
    rng = np.random.default_rng(int(seed))
    if allowed is None:
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    allowed = np.asarray(allowed, dtype=np.uint8)
    return allowed[rng.integers(0, len(allowed), size=shape)]


def all_bf16_patterns():
    """Every one of the 65536 bf16 bit patterns, in order."""
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)
