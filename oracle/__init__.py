"""Plain fp64 CPU oracle for block-hybrid attention (ctypes binding).

TEST INFRASTRUCTURE ONLY: the reference the HIP library is checked against.
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP library
and never imports it.

The arithmetic lives in ``bha_oracle.c`` (plain C, double precision, loops in
the order of the definitions); this module only loads it, checks shapes and
passes numpy arrays. Layouts (all C-contiguous float64):

* ``phi(x, w)``: x [n][d], w [FW][d] (row j = column j of the d x FW matrix W)
  -> phi [n][2FW] = [softmax(xW), softmax(-xW)] per token.
* ``state_build(k, v, w)`` -> (S [2FW][d], Z [2FW]).
* ``state_commit(S, Z, k, v, w)`` updates S, Z in place.
* ``block_forward(q, k, v, w, gamma, S, Z, scale)`` -> out [B][d].
* ``prefix_attention(q, k, v, kp, vp, scale)``: softmax attention of the
  block's queries over the whole prefix plus the block (the path the method
  replaces) -> out [B][d].
* batched variants over (request, head) pairs with plain pair-major layouts
  q/k/v/out [R][H][B][d], w [H][FW][d], gamma [H], S [R][H][2FW][d], Z [R][H][2FW].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bha_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libbha_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libbha_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _open(path: str):
    """Load an oracle library from ``path`` with its call signatures set."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.bha_ref_feature_map.argtypes = [I, I, I, P, P, P]
    lib.bha_ref_state_commit.argtypes = [I, I, I, P, P, P, P, P]
    lib.bha_ref_state_build.argtypes = [I, I, I, P, P, P, P, P]
    lib.bha_ref_block_forward.argtypes = [I, I, I, P, P, P, P, D, D, P, P, P]
    lib.bha_ref_block_forward_batch.argtypes = [I, I, I, I, I, P, P, P, P, P, D, P, P, P, I]
    lib.bha_ref_state_commit_batch.argtypes = [I, I, I, I, I, P, P, P, P, P, I]
    lib.bha_ref_prefix_attention.argtypes = [I, I, I, P, P, P, P, P, D, P]
    lib.bha_ref_prefix_attention.restype = None
    for f in (lib.bha_ref_feature_map, lib.bha_ref_state_commit, lib.bha_ref_state_build,
              lib.bha_ref_block_forward, lib.bha_ref_block_forward_batch,
              lib.bha_ref_state_commit_batch):
        f.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _open(_LIB_PATH)
    return _lib


def _f64(a, shape=None, name="array"):
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(a.shape)}")
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def phi(x, w):
    """Hedgehog feature map of every row of ``x`` ([n][d]) with ``w`` ([FW][d])."""
    w = _f64(w, name="w")
    fw, d = w.shape
    x = _f64(x, name="x")
    x2 = x.reshape(-1, d)
    out = np.empty((x2.shape[0], 2 * fw), dtype=np.float64)
    _load().bha_ref_feature_map(x2.shape[0], d, fw, _p(x2), _p(w), _p(out))
    return out.reshape(x.shape[:-1] + (2 * fw,))


def state_build(k, v, w):
    """(S, Z) of a prefix given all its keys/values ([N][d] each)."""
    w = _f64(w, name="w")
    fw, d = w.shape
    k = _f64(k, name="k").reshape(-1, d)
    v = _f64(v, (k.shape[0], d), "v")
    S = np.empty((2 * fw, d), dtype=np.float64)
    Z = np.empty((2 * fw,), dtype=np.float64)
    _load().bha_ref_state_build(k.shape[0], d, fw, _p(k), _p(v), _p(w), _p(S), _p(Z))
    return S, Z


def state_commit(S, Z, k, v, w):
    """In-place S += Phi(k)^T v, Z += sum Phi(k). S, Z must be float64 C-contiguous."""
    w = _f64(w, name="w")
    fw, d = w.shape
    if S.dtype != np.float64 or not S.flags.c_contiguous or S.shape != (2 * fw, d):
        raise ValueError("S must be a C-contiguous float64 [2FW][d] array")
    if Z.dtype != np.float64 or not Z.flags.c_contiguous or Z.shape != (2 * fw,):
        raise ValueError("Z must be a C-contiguous float64 [2FW] array")
    k = _f64(k, name="k").reshape(-1, d)
    v = _f64(v, (k.shape[0], d), "v")
    _load().bha_ref_state_commit(k.shape[0], d, fw, _p(k), _p(v), _p(w), _p(S), _p(Z))


def block_forward(q, k, v, w, gamma, S, Z, scale=0.0):
    """Block-hybrid forward of one (request, head): q, k, v [B][d] -> out [B][d]."""
    w = _f64(w, name="w")
    fw, d = w.shape
    q = _f64(q, name="q")
    B = q.shape[0]
    k = _f64(k, (B, d), "k")
    v = _f64(v, (B, d), "v")
    S = _f64(S, (2 * fw, d), "S")
    Z = _f64(Z, (2 * fw,), "Z")
    out = np.empty((B, d), dtype=np.float64)
    _load().bha_ref_block_forward(B, d, fw, _p(q), _p(k), _p(v), _p(w), float(gamma),
                                  float(scale), _p(S), _p(Z), _p(out))
    return out


def prefix_attention(q, k, v, kp, vp, scale=0.0):
    """Softmax attention of the block's queries over prefix + block keys:
    q, k, v [B][d], kp, vp [N][d] -> out [B][d]."""
    q = _f64(q, name="q")
    B, d = q.shape
    k = _f64(k, (B, d), "k")
    v = _f64(v, (B, d), "v")
    kp = _f64(kp, name="kp").reshape(-1, d)
    vp = _f64(vp, (kp.shape[0], d), "vp")
    out = np.empty((B, d), dtype=np.float64)
    _load().bha_ref_prefix_attention(B, kp.shape[0], d, _p(q), _p(k), _p(v), _p(kp), _p(vp),
                                     float(scale), _p(out))
    return out


def block_forward_batch(q, k, v, w, gamma, S, Z, scale=0.0, nthreads=1):
    """Every (request, head) pair: q/k/v [R][H][B][d] -> out [R][H][B][d]."""
    q = _f64(q, name="q")
    R, H, B, d = q.shape
    w = _f64(w, name="w")
    fw = w.shape[1]
    w = _f64(w, (H, fw, d), "w")
    k = _f64(k, (R, H, B, d), "k")
    v = _f64(v, (R, H, B, d), "v")
    gamma = _f64(gamma, (H,), "gamma")
    S = _f64(S, (R, H, 2 * fw, d), "S")
    Z = _f64(Z, (R, H, 2 * fw), "Z")
    out = np.empty((R, H, B, d), dtype=np.float64)
    _load().bha_ref_block_forward_batch(R, H, B, d, fw, _p(q), _p(k), _p(v), _p(w), _p(gamma),
                                        float(scale), _p(S), _p(Z), _p(out), int(nthreads))
    return out


def state_commit_batch(S, Z, k, v, w, nthreads=1):
    """Every (request, head) pair, in place: S [R][H][2FW][d], Z [R][H][2FW]."""
    k = _f64(k, name="k")
    R, H, B, d = k.shape
    w = _f64(w, name="w")
    fw = w.shape[1]
    w = _f64(w, (H, fw, d), "w")
    v = _f64(v, (R, H, B, d), "v")
    for a, shp, nm in ((S, (R, H, 2 * fw, d), "S"), (Z, (R, H, 2 * fw), "Z")):
        if a.dtype != np.float64 or not a.flags.c_contiguous or tuple(a.shape) != shp:
            raise ValueError(f"{nm} must be C-contiguous float64 of shape {shp}")
    _load().bha_ref_state_commit_batch(R, H, B, d, fw, _p(k), _p(v), _p(w), _p(S), _p(Z),
                                       int(nthreads))
