"""Helpers for the GPU parity tests: uploads, case announcements, metrics."""
import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def up(a, dtype=torch.float32):
    """numpy float32 array (values exactly representable in dtype) -> device."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    return t.to(dtype) if dtype != torch.float32 else t


def down(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits_down(t):
    return t.cpu().numpy().view(np.uint32)


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def bit_agreement(bits_a, bits_b, nbits):
    x = np.bitwise_xor(np.asarray(bits_a, dtype=np.uint32), np.asarray(bits_b, dtype=np.uint32))
    diff = int(np.unpackbits(x.view(np.uint8)).sum())
    return 1.0 - diff / float(nbits)


def empty_bits(rows, cin):
    return torch.empty((rows, cin // 32), dtype=torch.int32, device=DEV)
