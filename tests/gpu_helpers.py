"""Helpers for the GPU parity tests: move the generator's host arrays to the
device, call the library through its binding, bring results back."""
import sys

import numpy as np


def announce(msg: str) -> None:
    """Name the case before a GPU step so a crash log shows what was running."""
    sys.stderr.write(f"[gpu] {msg}\n")
    sys.stderr.flush()


def torch_mod():
    import torch
    return torch


def dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch = torch_mod()
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_rotq(twl, x_bits: np.ndarray, sign: np.ndarray):
    torch = torch_mod()
    x = dev(x_bits.view(np.int16))
    xi, sc = twl.rotate_quant_act(x, dev(sign))
    return host(xi), host(sc)


def gpu_pack(twl, code: np.ndarray, s_bits: np.ndarray, bad=None):
    packed, q, smax = twl.pack_ternary(dev(code), dev(s_bits.view(np.int16)), bad_codes=bad)
    return packed, q, smax


def gpu_linear(twl, x_i8, a_scale, packed, q, smax, path, out_acc):
    """x_i8, a_scale numpy; packed, q, smax device tensors (from the GPU pack)."""
    xi = dev(x_i8)
    if out_acc:
        return host(twl.ternary_linear_acc(xi, packed, q, path=path))
    return host(twl.ternary_linear(xi, dev(a_scale), packed, q, smax, path=path))
