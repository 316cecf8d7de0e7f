"""Seeded synthetic inputs: the only code the oracle side and the HIP side share.

It draws random tensors of the workloads' shapes and distributions and holds
none of the step's arithmetic.  Tensors are filled in place, chunk by chunk,
each chunk from its own ``torch.Generator`` seeded by (seed, stream, chunk),
so a value never depends on how many chunks came before it on another stream.

Distributions (the pages give none; these are the workloads' stated ones):
16-bit gradients ~ N(0, std) drawn by torch in the tensor's dtype, optionally
with a Bernoulli(frac) subset multiplied by ``mult``; fp32 master ~ N(0, std);
m ~ N(0, std); v = |N(0, std)|.
"""

import torch

CHUNK = 1 << 26            # elements per generator chunk
_GOLDEN = 0x9E3779B97F4A7C15
_MASK = (1 << 63) - 1

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


def stream_seed(seed, *keys):
    """Deterministic 63-bit seed for (seed, key, key, ...) -- a splitmix64 mix."""
    x = (seed * _GOLDEN) & ((1 << 64) - 1)
    for k in keys:
        x ^= (int(k) + _GOLDEN + (x << 6) + (x >> 2)) & ((1 << 64) - 1)
        x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9 & ((1 << 64) - 1)
        x = (x ^ (x >> 27)) * 0x94D049BB133111EB & ((1 << 64) - 1)
        x ^= x >> 31
    return x & _MASK


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _chunks(t):
    flat = t.view(-1)
    for ci, lo in enumerate(range(0, flat.numel(), CHUNK)):
        yield ci, flat[lo:lo + CHUNK]


def normal_(t, std, seed, stream, via=None):
    """Fill ``t`` with N(0, std) in its own dtype.

    With ``via`` (a device), each chunk is drawn there and copied into ``t``:
    a host tensor filled via the GPU holds the same values as a GPU tensor
    filled directly.
    """
    for ci, piece in _chunks(t):
        g = _gen(via if via is not None else t.device, stream_seed(seed, stream, ci))
        if via is None or torch.device(via).type == piece.device.type:
            piece.normal_(0.0, std, generator=g)
        else:
            tmp = torch.empty(piece.shape, dtype=piece.dtype, device=via)
            piece.copy_(tmp.normal_(0.0, std, generator=g))
    return t


def abs_normal_(t, std, seed, stream, via=None):
    """Fill ``t`` with |N(0, std)|."""
    normal_(t, std, seed, stream, via)
    return t.abs_()


def outliers_(t, frac, mult, seed, stream):
    """Multiply a Bernoulli(frac) subset of ``t`` by ``mult`` (in place)."""
    if frac <= 0:
        return t
    for ci, piece in _chunks(t):
        g = _gen(t.device, stream_seed(seed, stream, 1 << 20, ci))
        mask = torch.rand(piece.shape, device=t.device, generator=g) < frac
        piece[mask] *= mult
    return t


def tile_(t, period):
    """Repeat the first ``period`` elements of ``t`` over the whole tensor.

    A tiled vector's sum of squares is (whole periods) x (one period's) plus
    the partial tail, which lets a full-size norm be checked from one period.
    """
    flat = t.view(-1)
    n = flat.numel()
    done = min(period, n)
    while done < n:
        step = min(done, n - done)
        flat[done:done + step].copy_(flat[:step])
        done += step
    return t


def grad16(n, dtype, std, seed, stream, device, outlier_frac=0.0, outlier_mult=1.0):
    t = torch.empty(n, dtype=TORCH_DTYPES[dtype], device=device)
    normal_(t, std, seed, stream)
    return outliers_(t, outlier_frac, outlier_mult, seed, stream)


def state_f32(n, std, seed, stream, device, absolute=False):
    t = torch.empty(n, dtype=torch.float32, device=device)
    if std == 0:
        return t.zero_()
    return abs_normal_(t, std, seed, stream) if absolute else normal_(t, std, seed, stream)


def bits(t):
    """numpy uint16 view of a 16-bit tensor's bit patterns (copied to the host)."""
    import numpy as np
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
