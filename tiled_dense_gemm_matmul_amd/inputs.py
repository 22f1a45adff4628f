"""Seeded synthetic inputs for the forward GEMM family.

This module holds no arithmetic of the method: it only draws the operands
(activations ~ N(0, 1), weights ~ N(0, 0.02^2), f16 weights rounded to nearest
even from the fp32 draw) with the shapes of the workloads the pages describe:
sequence 512, d_model 768, d_ff 3072, vocabulary 16384 ("matmul ve
matmul_residual — Tiled Matrix Multiply (Forward)", section "Ne Yapar?"), and a
16 x 512-token batch with a 50304-entry vocabulary.  Both the HIP path and the
CPU oracle are fed the same host arrays produced here; no dataset or trained
weight is involved.

Draw order, per workload (numpy.random.default_rng(seed), float32 normals):

  cfg1  seed 0: X[128,768]; W[768,768]
  cfg2  seed 1: X[512,768]; W[768,768]; R[512,768]
  cfg3  seed 2: G[512,3072]; U[512,3072]; W[3072,768]; R[512,768]; then
                1 % of G (15728 positions, drawn without replacement) set to
                +-80 with a fair-coin sign
  cfg4  seed 3: X[512,768]; W_lm[768,16384] -> f16; W_gu[768,3072] -> f16
  cfg5  seed 4: G[8192,3072]; U[8192,3072]; W_down[3072,768] -> f16;
                R[8192,768]; X[8192,768]; W_lm[768,50304] -> f16
"""
from __future__ import annotations

import numpy as np

W_STD = np.float32(0.02)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _weight(rng, shape):
    return _normal(rng, shape) * W_STD


def cfg1():
    rng = np.random.default_rng(0)
    X = _normal(rng, (128, 768))
    W = _weight(rng, (768, 768))
    return {"X": X, "W": W}


def cfg2():
    rng = np.random.default_rng(1)
    X = _normal(rng, (512, 768))
    W = _weight(rng, (768, 768))
    R = _normal(rng, (512, 768))
    return {"X": X, "W": W, "R": R}


def gate_outliers(rng, G, frac=0.01, magnitude=80.0):
    """Set floor(frac * G.size) distinct positions of G to +-magnitude (in place)."""
    count = int(np.floor(frac * G.size))
    idx = rng.permutation(G.size)[:count]
    sign = 2 * rng.integers(0, 2, count) - 1
    G.reshape(-1)[idx] = (magnitude * sign).astype(np.float32)
    return idx


def cfg3():
    rng = np.random.default_rng(2)
    G = _normal(rng, (512, 3072))
    U = _normal(rng, (512, 3072))
    W = _weight(rng, (3072, 768))
    R = _normal(rng, (512, 768))
    gate_outliers(rng, G)
    return {"G": G, "U": U, "W": W, "R": R}


def cfg4():
    rng = np.random.default_rng(3)
    X = _normal(rng, (512, 768))
    W_lm = _weight(rng, (768, 16384)).astype(np.float16)
    W_gu = _weight(rng, (768, 3072)).astype(np.float16)
    return {"X": X, "W_lm": W_lm, "W_gu": W_gu}


def cfg5():
    rng = np.random.default_rng(4)
    G = _normal(rng, (8192, 3072))
    U = _normal(rng, (8192, 3072))
    W_down = _weight(rng, (3072, 768)).astype(np.float16)
    R = _normal(rng, (8192, 768))
    X = _normal(rng, (8192, 768))
    W_lm = _weight(rng, (768, 50304)).astype(np.float16)
    return {"G": G, "U": U, "W_down": W_down, "R": R, "X": X, "W_lm": W_lm}


def random_case(seed, M, K, N, *, swiglu=False, w16=False, residual=False,
                gate_scale=1.0, integer=False):
    """A generic seeded case of arbitrary shape (edge and ragged tests).

    integer=True draws small integers (|x| <= 8) so that every partial sum is
    exactly representable in fp32 for K <= 3072.
    """
    rng = np.random.default_rng(seed)
    if integer:
        def act(shape):
            return rng.integers(-8, 9, size=shape).astype(np.float32)
        def wt(shape):
            return rng.integers(-8, 9, size=shape).astype(np.float32)
    else:
        def act(shape):
            return _normal(rng, shape)
        def wt(shape):
            return _weight(rng, shape)
    out = {}
    if swiglu:
        out["G"] = act((M, K)) * np.float32(gate_scale)
        out["U"] = act((M, K))
    else:
        out["X"] = act((M, K))
    W = wt((K, N))
    out["W"] = W.astype(np.float16) if w16 else W
    if residual:
        out["R"] = act((M, N))
    return out


def backward_case(seed, M, K, N, *, swiglu=False, acc=False, gate_scale=1.0):
    """A seeded case for the backward products (forward names: M rows, K
    inputs, N outputs): X [M, K] (or GATE and UP), the forward weight W [K, N],
    the output gradient dY [M, N], and, for the accumulating forms, previous
    output contents dX0 [M, K] and dW0 [K, N]."""
    rng = np.random.default_rng(seed)
    out = {}
    if swiglu:
        out["G"] = _normal(rng, (M, K)) * np.float32(gate_scale)
        out["U"] = _normal(rng, (M, K))
    else:
        out["X"] = _normal(rng, (M, K))
    out["W"] = _weight(rng, (K, N))
    out["dY"] = _normal(rng, (M, N))
    if acc:
        out["dX0"] = _normal(rng, (M, K))
        out["dW0"] = _normal(rng, (K, N))
    return out


def loss_case(seed, S, V, *, scale=2.0, ignore_every=0):
    """A seeded case for the fused loss: logits [S, V] float32 drawn N(0, 1)
    times `scale`, targets [S] uint32 uniform in [0, V); with ignore_every =
    k > 0 every k-th row gets the ignored target V (padding)."""
    rng = np.random.default_rng(seed)
    logits = _normal(rng, (S, V)) * np.float32(scale)
    targets = rng.integers(0, max(V, 1), size=S).astype(np.uint32) if V > 0 else np.zeros(S, np.uint32)
    if ignore_every:
        targets[::ignore_every] = V
    return {"logits": logits, "targets": targets}


def activation_case(seed, n, *, scale=3.0):
    """A seeded case for the FFN activation kernels: the hidden gradient g,
    gate (also used as the GeLU input) and up, n float32 values each; gate is
    drawn N(0, 1) times `scale` so both tails of the sigmoid and of tanh are
    exercised."""
    rng = np.random.default_rng(seed)
    return {"g": _normal(rng, (n,)), "gate": _normal(rng, (n,)) * np.float32(scale), "up": _normal(rng, (n,))}
