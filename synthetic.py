"""Seeded synthetic inputs for the W4A16 GEMV (shared by tests, smoke and bench).

This module only draws random numbers; it holds none of the method's
arithmetic (no packing, no dequantization, no products). Both the oracle and
the HIP path receive what it returns.

Distributions (the workload definition of this project):
  q  uniform integers 0..15,                      uint8  [N][K]
  s  |N(0, 0.02)| + 1e-3, rounded to fp16 (RNE),  uint16 fp16 bits [N][K/128]
  z  uniform integers 0..15,                      uint8  [N][K/128]
  x  N(0, 1), rounded to fp16 (RNE),              uint16 fp16 bits [M][K]

Every tensor has its own stream: numpy's PCG64 seeded with
SeedSequence([seed, tensor_id, stream]), so a tensor never depends on which
other tensors were drawn before it.
"""
import numpy as np

GROUP = 128

_Q, _S, _Z, _X, _BYTES = 1, 2, 3, 4, 5


def _rng(seed, tensor_id, stream):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id), stream])))


def weights(N, K, seed=0, tensor_id=0):
    """Logical (q, s, z) for an N x K weight matrix."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    G = K // GROUP
    q = _rng(seed, tensor_id, _Q).integers(0, 16, size=(N, K), dtype=np.uint8)
    sv = np.abs(_rng(seed, tensor_id, _S).normal(0.0, 0.02, size=(N, G))) + 1e-3
    s = sv.astype(np.float16).view(np.uint16)
    z = _rng(seed, tensor_id, _Z).integers(0, 16, size=(N, G), dtype=np.uint8)
    return q, s, z


def activations(M, K, seed=0, tensor_id=0):
    """fp16 bits of x [M][K] ~ N(0, 1)."""
    xv = _rng(seed, tensor_id, _X).normal(0.0, 1.0, size=(M, K))
    return xv.astype(np.float16).view(np.uint16)


def uniform_bytes(nbytes, seed=0, tensor_id=0):
    """Independent uniform bytes. Two uniform 4-bit values per byte have the
    same joint law as uniform q (or z) written two to a byte in any fixed
    order, so large benchmark weight buffers can be drawn in packed form."""
    return np.frombuffer(_rng(seed, tensor_id, _BYTES).bytes(int(nbytes)), dtype=np.uint8)


def scales(N, G, seed=0, tensor_id=0):
    """Only the fp16 scale bits [N][G] (same law and stream as weights())."""
    sv = np.abs(_rng(seed, tensor_id, _S).normal(0.0, 0.02, size=(N, G))) + 1e-3
    return sv.astype(np.float16).view(np.uint16)


# Workload shapes (N x K at M rows), named by what they are.
QWEN05B_LAYER = [("q_proj", 896, 896), ("k_proj", 128, 896), ("v_proj", 128, 896),
                 ("o_proj", 896, 896), ("gate_proj", 4864, 896), ("up_proj", 4864, 896),
                 ("down_proj", 896, 4864)]
QWEN05B_LAYERS = 24

QWEN7B_LAYER = [("qkv_proj", 4608, 3584), ("o_proj", 3584, 3584),
                ("gate_up_proj", 37888, 3584), ("down_proj", 3584, 18944)]
QWEN7B_LAYERS = 28
QWEN7B_LM_HEAD = ("lm_head", 152064, 3584)

VERIFY27B = [("up_27b", 17408, 5120), ("down_27b", 5120, 17408)]
VERIFY_M = (1, 2, 5, 8)

SINGLE_896 = ("single_896", 896, 896)



def device_packed_weights(N, K, seed, tensor_id, device):
    """Weights drawn directly in layout-ID-2 form on the GPU (for large
    benchmark sets, where drawing logical q on the host would dominate).

    Same law as packing weights(): packed nibbles of uniform q (and z) are
    uniform random bytes; scales are fp16(|N(0, 0.02)| + 1e-3) in every
    (row, group) slot, padding rows included (their outputs are never stored).
    Uses torch's seeded device generator. Returns (wq, scales, zeros) as
    uint8/int16/uint8 torch tensors of the packed sizes."""
    import torch
    NP = (N + 15) // 16 * 16
    G = K // GROUP
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + int(tensor_id))
    wq = torch.randint(0, 256, (NP * K // 2,), dtype=torch.uint8, device=device, generator=gen)
    sv = torch.randn((NP * G,), dtype=torch.float32, device=device, generator=gen).mul_(0.02).abs_().add_(1e-3)
    sc = sv.to(torch.float16).view(torch.int16).reshape(-1)
    zp = torch.randint(0, 256, (NP * G // 2,), dtype=torch.uint8, device=device, generator=gen)
    return wq, sc, zp


def device_activations(M, K, seed, tensor_id, device):
    """fp16 x [M][K] ~ N(0, 1) drawn on the GPU (int16 view of the bits)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 500009 + int(tensor_id))
    return torch.randn((M, K), dtype=torch.float32, device=device, generator=gen).to(torch.float16).view(torch.int16)
