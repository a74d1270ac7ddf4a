"""Helpers for the GPU parity tests: moving seeded bf16 bit patterns between
numpy (oracle side) and torch device tensors (library side).  No arithmetic of
the method lives here."""
import numpy as np
import torch


def dev_bf16(u16):
    """uint16 bf16 bits (numpy) -> contiguous torch.bfloat16 tensor on cuda:0."""
    a = np.ascontiguousarray(u16, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")


def host_bits(t):
    """torch.bfloat16 tensor -> uint16 numpy bits."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t):
    """bf16 / fp32 tensor -> float64 numpy (exact)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def say(msg):
    print(msg, flush=True)


def dev_f16(u16):
    """uint16 fp16 bits (numpy) -> contiguous torch.float16 tensor on cuda:0."""
    a = np.ascontiguousarray(u16, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.float16).to("cuda:0")


def dev_f32(u32):
    """uint32 fp32 bits (numpy) -> contiguous torch.float32 tensor on cuda:0."""
    a = np.ascontiguousarray(u32, dtype=np.uint32)
    return torch.from_numpy(a.view(np.float32)).to("cuda:0")


def host_bits32(t):
    """torch.float32 tensor -> uint32 numpy bits."""
    return t.detach().cpu().numpy().view(np.uint32)
