"""Test inputs that enumerate the quantizer's per-element domain.

Under 1x128 / 128x128 quantization every code is a function of just two bf16 numbers: the
element x and its group's amax (|x| <= amax).  ``domain_tiles`` lays out, for each
requested amax, every bf16 x with |x| <= amax (both signs, both zeros) in 1x128 tiles whose
element 0 is amax itself, so each tile's amax is exactly that value.  Pure input layout:
no quantization arithmetic.
"""
import numpy as np


def domain_tiles(amax_bits):
    """Return (X bits [T,128] uint16, amax bits per tile [T], count of real x per tile [T])."""
    rows, amaxes, counts = [], [], []
    for a in np.asarray(amax_bits, dtype=np.int64):
        xs = np.concatenate([np.arange(0, a + 1), 0x8000 + np.arange(0, a + 1)]).astype(np.uint16)
        n = xs.size
        t = (n + 126) // 127
        body = np.zeros(t * 127, dtype=np.uint16)
        body[:n] = xs
        tiles = np.empty((t, 128), dtype=np.uint16)
        tiles[:, 0] = a
        tiles[:, 1:] = body.reshape(t, 127)
        cnt = np.full(t, 127, dtype=np.int64)
        cnt[-1] = n - 127 * (t - 1)
        rows.append(tiles)
        amaxes.append(np.full(t, a, dtype=np.uint16))
        counts.append(cnt)
    return np.concatenate(rows), np.concatenate(amaxes), np.concatenate(counts)


def all_amax_bits():
    """Every positive finite bf16 amax (0x0001 .. 0x7F7F)."""
    return np.arange(1, 0x7F80, dtype=np.int64)


def sampled_amax_bits(stride=61):
    """All bf16 subnormal amax values, a stride through the rest, and the edges."""
    a = set(range(1, 0x80)) | set(range(0x80, 0x7F80, stride))
    a |= {0x0080, 0x3F80, 0x4000, 0x43E0, 0x7F00, 0x7F7F, 0x0100, 0x00FF}
    return np.array(sorted(a), dtype=np.int64)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
