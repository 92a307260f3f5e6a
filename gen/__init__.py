"""Seeded synthetic inputs for the routed NVFP4 W4A4 MoE layer.

Serves both the oracle and the GPU path; holds none of the layer's arithmetic.
Every tensor is a pure function of (seed, config, layer, tensor id, step) through
counter-based SplitMix64 streams implemented in ``gen.c``.

Workload shapes follow the pages' model: 512 experts with 10 routed plus 1 shared
per layer (capy-flash README, "What it does" and the synthetic test-artifact
script; Richland article, "What shipped"), at hidden 2048 / expert intermediate
512.  Seed 1234 is the seed of the pages' synthetic test artifact.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libgen.so")

BASE_SEED = 1234
TENSOR_HIDDEN, TENSOR_ROUTER, TENSOR_W13, TENSOR_W2, TENSOR_SH13, TENSOR_SH2, TENSOR_SHGATE = range(7)


def build(force: bool = True) -> str:
    """Compile gen.c into libgen.so (gcc, OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", os.path.join(_HERE, "gen.c"),
                               "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.gen_splitmix64.argtypes = [u64, u64]
        L.gen_splitmix64.restype = u64
        L.gen_normal_at.argtypes = [u64, u64]
        L.gen_normal_at.restype = dbl
        L.gen_normal_bf16.argtypes = [u64, dbl, i64, vp]
        L.gen_normal_f32_rows.argtypes = [u64, vp, i64, i64, vp]
        L.gen_nvfp4_bank.argtypes = [u64, dbl, i64, i64, i64, vp, vp, vp]
        L.gen_nvfp4_bank.restype = ctypes.c_int
        _lib = L
    return _lib


def _mix(z: int) -> int:
    m = (1 << 64) - 1
    z &= m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def stream_key(seed: int, cfg: int, layer: int, tensor: int, step: int = 0) -> int:
    """Key of one tensor's SplitMix64 stream."""
    k = _mix(seed)
    for part in (cfg, layer, tensor, step):
        k = _mix(k ^ (_mix(part + 0x51ED27) & ((1 << 64) - 1)))
    return k


@dataclass(frozen=True)
class Shape:
    H: int
    E: int
    k: int
    I: int


SHAPES = {0: Shape(256, 16, 2, 128), 1: Shape(2048, 512, 10, 512), 2: Shape(2048, 512, 10, 512),
          3: Shape(2048, 512, 10, 512), 4: Shape(2048, 512, 10, 512)}
# token counts per config; config 4 is 48 layers of the config-1 shape
TOKENS = {0: (8,), 1: (1, 4), 2: (4096,), 3: (15360,), 4: (1, 4, 4096)}
ZIPF_CONFIGS = (2, 3)
WEIGHT_SIGMA = 0.02
ROUTER_SIGMA = 0.02


def normal_bf16(key: int, n: int, scale: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().gen_normal_bf16(key, scale, n, out.ctypes.data)
    return out


def normal_f32_rows(key: int, row_scale: np.ndarray, cols: int) -> np.ndarray:
    rs = np.ascontiguousarray(row_scale, dtype=np.float64)
    out = np.empty((rs.shape[0], cols), dtype=np.float32)
    lib().gen_normal_f32_rows(key, rs.ctypes.data, rs.shape[0], cols, out.ctypes.data)
    return out


def nvfp4_bank(key: int, n_exp: int, N: int, K: int, sigma: float = WEIGHT_SIGMA) -> dict:
    """[n_exp][N][K] N(0, sigma^2) weights packed as NVFP4 (codes, scales, gscale)."""
    codes = np.empty((n_exp, N, K // 2), dtype=np.uint8)
    scales = np.empty((n_exp, N, K // 16), dtype=np.uint8)
    gscale = np.empty(n_exp, dtype=np.float32)
    rc = lib().gen_nvfp4_bank(key, sigma, n_exp, N, K, codes.ctypes.data, scales.ctypes.data, gscale.ctypes.data)
    if rc != 0:
        raise RuntimeError("gen_nvfp4_bank failed: %d" % rc)
    return {"codes": codes, "scales": scales, "gscale": gscale}


def zipf_targets(E: int, k: int, s: float = 1.1, cap: float = 0.5) -> np.ndarray:
    """Per-rank selection probabilities p_r = min(cap, c * r^-s) with sum k (water-filled).

    A bias-free linear router fed zero-mean symmetric tokens cannot put an expert
    in the top k of more than half the tokens (x -> -x swaps top and bottom), so
    the head of the Zipf law is capped at 1/2 and the mass is refilled below it.
    """
    r = np.arange(1, E + 1, dtype=np.float64)
    base = r ** (-s)
    lo, hi = 0.0, 1e6
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(cap, c * base).sum() > k:
            hi = c
        else:
            lo = c
    return np.minimum(cap, 0.5 * (lo + hi) * base)


def zipf_router_sigmas(seed: int, cfg: int, layer: int, E: int, k: int, H: int, z_norms: np.ndarray,
                       n_sim: int = 8192, rounds: int = 24) -> tuple[np.ndarray, np.ndarray]:
    """Row multipliers sigma_e that make top-k membership follow the capped Zipf law.

    Logits are modelled as independent N(0, (sigma_e*|z_e|)^2) (random rows in
    H dimensions are nearly orthogonal); sigma is refined multiplicatively on a
    fixed set of simulated tokens.  Returns (sigma per expert id, target p per expert id).
    """
    rng = np.random.default_rng(stream_key(seed, cfg, layer, TENSOR_ROUTER, 1) & ((1 << 63) - 1))
    perm = rng.permutation(E)  # perm[rank] = expert id
    target = np.empty(E)
    target[perm] = zipf_targets(E, k)
    z = rng.standard_normal((n_sim, E))
    sig = np.ones(E)
    for _ in range(rounds):
        std = sig * z_norms
        lg = z * std[None, :]
        top = np.argpartition(-lg, k - 1, axis=1)[:, :k]
        p = np.bincount(top.ravel(), minlength=E) / n_sim
        sig = sig * (target / np.maximum(p, 0.5 / n_sim)) ** 0.3
        sig = np.minimum(sig, 50.0 * np.median(sig))
        sig = sig / np.exp(np.mean(np.log(sig)))
    return sig, target


def router_weights(seed: int, cfg: int, layer: int, shape: Shape) -> np.ndarray:
    key = stream_key(seed, cfg, layer, TENSOR_ROUTER)
    if cfg not in ZIPF_CONFIGS:
        return normal_f32_rows(key, np.full(shape.E, ROUTER_SIGMA), shape.H)
    z = normal_f32_rows(key, np.full(shape.E, ROUTER_SIGMA), shape.H)
    norms = np.sqrt((z.astype(np.float64) ** 2).sum(axis=1))
    sig, _ = zipf_router_sigmas(seed, cfg, layer, shape.E, shape.k, shape.H, norms)
    return normal_f32_rows(key, ROUTER_SIGMA * sig, shape.H)


@dataclass
class Layer:
    shape: Shape
    router_w: np.ndarray  # [E][H] f32
    w13: dict  # codes [E][2I][H/2], scales [E][2I][H/16], gscale [E]
    w2: dict   # codes [E][H][I/2], scales [E][H][I/16], gscale [E]
    sh13: dict  # n_exp = 1
    sh2: dict
    a_gscale_in: float = 1.0
    a_gscale_mid: float = 1.0
    shared_gate_w: np.ndarray | None = None  # [H] f32, optional gate of the shared expert
    act_bits: int = 4  # activation encoding: 4 (W4A4) or 8 (the W4A8 variant)


def make_layer(cfg: int, layer: int = 0, seed: int = BASE_SEED, shape: Shape | None = None,
               shared_gate: bool = False) -> Layer:
    """One MoE layer's weights (router FP32, routed and shared NVFP4 banks, and with
    shared_gate an N(0, 0.02^2) FP32 gate vector for the shared expert)."""
    sh = shape or SHAPES[cfg]
    sk = lambda t: stream_key(seed, cfg, layer, t)
    return Layer(
        shape=sh,
        router_w=router_weights(seed, cfg, layer, sh),
        w13=nvfp4_bank(sk(TENSOR_W13), sh.E, 2 * sh.I, sh.H),
        w2=nvfp4_bank(sk(TENSOR_W2), sh.E, sh.H, sh.I),
        sh13=nvfp4_bank(sk(TENSOR_SH13), 1, 2 * sh.I, sh.H),
        sh2=nvfp4_bank(sk(TENSOR_SH2), 1, sh.H, sh.I),
        shared_gate_w=normal_f32_rows(sk(TENSOR_SHGATE), np.array([ROUTER_SIGMA]), sh.H)[0] if shared_gate else None,
    )


def make_tokens(cfg: int, T: int, step: int = 0, layer: int = 0, seed: int = BASE_SEED, H: int | None = None
                ) -> np.ndarray:
    """[T][H] BF16 bit patterns of N(0,1) hidden states; `step` selects a fresh batch."""
    H = H or SHAPES[cfg].H
    return normal_bf16(stream_key(seed, cfg, layer, TENSOR_HIDDEN, step), T * H).reshape(T, H)
