"""Seeded synthetic inputs, and their storage encodings (no step of the method).

Every tensor of a workload is drawn from its own torch generator seeded with
    seed * 1_000_003 + 1000 * workload_id + tensor_id
on the device that will hold it, then encoded to its storage format:
  * bf16 by torch's round-to-nearest-even cast;
  * fp8 rows: OCP e4m3fn codes with one fp32 scale per row, s = max|row|/448;
  * MXFP4: e2m1 codes (round to nearest, ties to the even code, saturating at
    6) with one E8M0 scale per 32 elements, exponent floor(log2 max|block|) - 2
    clipped to [-3, 0] so that every indexer score stays exact in fp32.
Both the HIP path (through the tests and the benchmark) and the oracle (on a
host copy) consume these tensors; this module computes nothing of the method.
"""
import math

import torch

MX_EXP_MIN, MX_EXP_MAX = -3, 0
_E2M1_MIDS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def seed_of(seed, workload_id, tensor_id):
    return seed * 1_000_003 + 1000 * workload_id + tensor_id


def generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std, seed, device, dtype=torch.float32):
    g = generator(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def normal_bf16_bits(shape, std, seed, device, chunk_elems=1 << 28):
    """N(0, std^2) rounded to bf16, returned as int16 bit patterns; drawn in chunks along dim 0..1."""
    out = torch.empty(shape, dtype=torch.int16, device=device)
    g = generator(seed, device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        x.mul_(std)
        flat[s:e] = x.to(torch.bfloat16).view(torch.int16)
    return out


def bf16_bits(x):
    return x.to(torch.bfloat16).view(torch.int16)


def fp8_rows(x):
    """x [..., D] fp32 -> (codes uint8 [..., D], scale fp32 [...]) with s = max|row| / 448 (1 if 0)."""
    amax = x.abs().amax(dim=-1)
    s = amax / 448.0
    s = torch.where(amax == 0, torch.ones_like(s), s)
    codes = (x / s.unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, s.to(torch.float32)


def mxfp4(x, e_min=MX_EXP_MIN, e_max=MX_EXP_MAX):
    """x [..., D] fp32 (D % 32 == 0) -> (packed uint8 [..., D/2], scale E8M0 uint8 [..., D/32]);
    block exponents limited to [e_min, e_max] (indexer vectors: [-3, 0])."""
    D = x.shape[-1]
    assert D % 32 == 0
    xb = x.reshape(*x.shape[:-1], D // 32, 32)
    amax = xb.abs().amax(dim=-1, keepdim=True)
    e = torch.floor(torch.log2(torch.clamp(amax, min=2.0 ** -30))) - 2
    e = torch.clamp(e, e_min, e_max)
    mag = (xb.abs() / torch.exp2(e)).reshape(*x.shape[:-1], D)
    mids = torch.tensor(_E2M1_MIDS, device=x.device, dtype=torch.float32)
    lower = torch.bucketize(mag, mids, right=False)                   # ties -> lower code
    tie = (mag == mids[torch.clamp(lower, max=6)]) & (lower % 2 == 1)   # ... unless it is odd
    code = (lower + tie.to(lower.dtype)).to(torch.uint8)
    code = code | torch.where(x < 0, 8, 0).to(torch.uint8)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    scale = (e.squeeze(-1) + 127).to(torch.uint8)
    return packed.contiguous(), scale.contiguous()


def mxfp4_normal(shape, seed, device, chunk_rows=1 << 20):
    """N(0,1) drawn then MXFP4-encoded, in chunks of rows (shape [..., D])."""
    *lead, D = shape
    rows = math.prod(lead)
    packed = torch.empty(rows, D // 2, dtype=torch.uint8, device=device)
    scale = torch.empty(rows, D // 32, dtype=torch.uint8, device=device)
    g = generator(seed, device)
    for s in range(0, rows, chunk_rows):
        e = min(rows, s + chunk_rows)
        x = torch.randn(e - s, D, generator=g, device=device, dtype=torch.float32)
        packed[s:e], scale[s:e] = mxfp4(x)
    return packed.view(*lead, D // 2), scale.view(*lead, D // 32)


def mxfp4_rows_normal(shape, std, seed, device, chunk_rows=1 << 18):
    """N(0, std^2) rows -> MXFP4 KV entries (codes [..., D/2], E8M0 [..., D/32], exponents over the
    whole E8M0 range), in chunks of rows."""
    *lead, D = shape
    rows = math.prod(lead)
    packed = torch.empty(rows, D // 2, dtype=torch.uint8, device=device)
    scale = torch.empty(rows, D // 32, dtype=torch.uint8, device=device)
    g = generator(seed, device)
    for s in range(0, rows, chunk_rows):
        e = min(rows, s + chunk_rows)
        x = torch.randn(e - s, D, generator=g, device=device, dtype=torch.float32) * std
        packed[s:e], scale[s:e] = mxfp4(x, -127, 127)
    return packed.view(*lead, D // 2), scale.view(*lead, D // 32)


def fp8_rows_normal(shape, std, seed, device, chunk_rows=1 << 18):
    """N(0, std^2) rows -> per-row e4m3fn codes and fp32 scales, in chunks of rows."""
    *lead, D = shape
    rows = math.prod(lead)
    codes = torch.empty(rows, D, dtype=torch.uint8, device=device)
    scale = torch.empty(rows, dtype=torch.float32, device=device)
    g = generator(seed, device)
    for s in range(0, rows, chunk_rows):
        e = min(rows, s + chunk_rows)
        x = torch.randn(e - s, D, generator=g, device=device, dtype=torch.float32) * std
        codes[s:e], scale[s:e] = fp8_rows(x)
    return codes.view(*lead, D), scale.view(*lead)
