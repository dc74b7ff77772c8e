"""Seeded synthetic inputs for the OIDN-style UNet denoiser.

This module only draws random numbers: it holds no step of the method.  Both
the oracle-side tests and the HIP-side tests/benchmark take their inputs from
here, so the two sides see identical host arrays.

Recipe (numpy ``default_rng(seed)``; draw order is fixed: images first, then
for each layer its weights and then its bias):

* auxiliary images are RGBA float32, 16 bytes per pixel, row-major (H, W, 4);
* color: rgb lognormal(0, 1) (a stand-in for rendered HDR radiance), alpha
  uniform[0, 1];
* albedo: rgba uniform[0, 1];
* normal: 3-D standard normal vectors scaled to unit length (components in
  [-1, 1]), fourth lane 0;
* weights: He-normal, std sqrt(2 / (9 * Cin_logical)), OHWI float32;
* bias: normal(0, 0.01), float32.
"""
from __future__ import annotations

import numpy as np


def rng(seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(seed)


def images(r: np.random.Generator, width: int, height: int):
    """Color, albedo and normal RGBA float32 images of shape (height, width, 4)."""
    color = np.empty((height, width, 4), np.float32)
    color[..., :3] = np.exp(r.standard_normal((height, width, 3))).astype(np.float32)
    color[..., 3] = r.uniform(0.0, 1.0, (height, width)).astype(np.float32)
    albedo = r.uniform(0.0, 1.0, (height, width, 4)).astype(np.float32)
    n = r.standard_normal((height, width, 3))
    n /= np.maximum(np.linalg.norm(n, axis=-1, keepdims=True), 1e-12)
    normal = np.zeros((height, width, 4), np.float32)
    normal[..., :3] = n.astype(np.float32)
    return color, albedo, normal


def he_normal(r: np.random.Generator, cout: int, cin: int):
    """OHWI (cout, 3, 3, cin) float32 weights with std sqrt(2 / (9 * cin))."""
    std = np.sqrt(2.0 / (9.0 * cin))
    return (r.standard_normal((cout, 3, 3, cin)) * std).astype(np.float32)


def bias(r: np.random.Generator, cout: int):
    return r.normal(0.0, 0.01, cout).astype(np.float32)


def layer_params(r: np.random.Generator, shapes):
    """Weights and biases for a list of (cin_logical, cout) shapes, in order."""
    ws, bs = [], []
    for cin, cout in shapes:
        ws.append(he_normal(r, cout, cin))
        bs.append(bias(r, cout))
    return ws, bs


def uniform_activation(r: np.random.Generator, height: int, width: int, channels: int,
                       stored_channels: int):
    """(H, W, stored) float32, uniform[0, 1] in the first ``channels`` lanes, 0 after."""
    x = np.zeros((height, width, stored_channels), np.float32)
    x[..., :channels] = r.uniform(0.0, 1.0, (height, width, channels)).astype(np.float32)
    return x


def relu_normal_activation(r: np.random.Generator, height: int, width: int, channels: int,
                           stored_channels: int):
    """(H, W, stored) float32, max(0, N(0, 1)) in the first ``channels`` lanes, 0 after."""
    x = np.zeros((height, width, stored_channels), np.float32)
    x[..., :channels] = np.maximum(r.standard_normal((height, width, channels)), 0.0)
    return x
