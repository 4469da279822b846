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
    """Oracle products for all rows, or for `rows` only (those rows are packed on
    their own, which keeps full-size cases cheap; placement does not change
    what a row computes)."""
    if rows is None:
        cp, sp = oracle.pack(layer.codes, layer.scales)
        return oracle.linear(cp, sp, layer.codebook, layer.n, layer.k, x_bits)
    rows = np.asarray(rows)
    cp, sp = oracle.pack(layer.codes[rows], layer.scales[rows])
    return oracle.linear(cp, sp, layer.codebook[rows], len(rows), layer.k, x_bits)


def assert_close(y_gpu, y_ref, bound, what=""):
    ok, ratio = oracle.within_tolerance(y_gpu, y_ref, bound, rel=1e-3)
    assert ok, f"{what}: max |y - y_ref| / sum|x w| = {ratio:.3e} exceeds 1e-3"
    return ratio
