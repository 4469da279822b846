"""Helpers for the GPU parity tests: move seeded inputs to the device, pack them
with the library's q3_pack, and compute the oracle's expected values from the
same host arrays (the oracle never sees anything the GPU produced)."""
import numpy as np
import torch

import oracle


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def pack_layer(q3, layer):
    return q3.q3_pack(dev(layer.codes), dev(layer.scales), dev(layer.codebook))


def oracle_linear(layer, x_bits, rows=None):
    cp, sp = oracle.pack(layer.codes, layer.scales)
    return oracle.linear(cp, sp, layer.codebook, layer.n, layer.k, x_bits, rows=rows)


def assert_close(y_gpu, y_ref, bound, what=""):
    ok, ratio = oracle.within_tolerance(y_gpu, y_ref, bound, rel=1e-3)
    assert ok, f"{what}: max |y - y_ref| / sum|x w| = {ratio:.3e} exceeds 1e-3"
    return ratio
