"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module draws random tensors and nothing else: it contains no step of
the attention method.  Both sides of every parity check receive the exact
bytes produced here.  The generator itself is the C file ``synth.c`` beside
this module (SplitMix64 counter-based streams, Box-Muller normals, Floyd
sampling), compiled to ``libsynth.so`` with gcc and OpenMP.

Every tensor is a pure function of (seed, workload id, tensor id, element
index), so ``rows()`` can regenerate any slice of a tensor on its own, e.g.
the few latent-cache rows a sampled oracle check needs out of 4.5 GiB.

Storage dtypes: bf16 tensors are numpy ``uint16`` arrays holding bf16 bit
patterns, fp32 tensors are ``float32``, index tensors are ``int32``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

SYN_NORMAL, SYN_INT, SYN_POW2, SYN_CHOICE = 0, 1, 2, 3
SYN_F32, SYN_BF16 = 0, 1

TENSOR_IDS = {"q_idx": 1, "k_idx": 2, "w": 3, "q": 4, "kv": 5, "idx": 6}


def build_library(force: bool = False) -> str:
    """Compile synth.c into libsynth.so next to this file."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_library()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_stream_key.restype = ctypes.c_uint64
        lib.synth_stream_key.argtypes = [ctypes.c_uint64] * 3
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p]
        lib.synth_floyd.restype = ctypes.c_int
        lib.synth_floyd.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_void_p]
        _lib = lib
    return _lib


def stream_key(seed: int, workload_id: int, tensor_id: int) -> int:
    return int(_load().synth_stream_key(seed, workload_id, tensor_id))


@dataclass(frozen=True)
class Dist:
    """One tensor's value distribution: kind in normal/int/pow2/choice."""
    kind: str
    lo: int = 0
    hi: int = 0
    values: tuple = ()


def fill(key: int, start: int, count: int, dist: Dist, dtype: str) -> np.ndarray:
    """Elements [start, start+count) of the stream `key` under `dist`."""
    lib = _load()
    out = np.empty(count, dtype=np.uint16 if dtype == "bf16" else np.float32)
    kind = {"normal": SYN_NORMAL, "int": SYN_INT, "pow2": SYN_POW2, "choice": SYN_CHOICE}[dist.kind]
    vals = np.asarray(dist.values if dist.values else (0.0,), dtype=np.float64)
    rc = lib.synth_fill(key, start, count, kind, dist.lo, dist.hi,
                        vals.ctypes.data, len(dist.values), SYN_BF16 if dtype == "bf16" else SYN_F32,
                        out.ctypes.data)
    if rc != 0:
        raise ValueError("synth_fill rejected its arguments")
    return out


def floyd(key: int, rows: int, n: int, k: int) -> np.ndarray:
    out = np.empty((rows, k), dtype=np.int32)
    if _load().synth_floyd(key, rows, n, k, out.ctypes.data) != 0:
        raise ValueError("synth_floyd rejected its arguments")
    return out


@dataclass(frozen=True)
class Workload:
    """Shapes, value recipe and stages of one synthetic DSA workload.

    B sequences, Tq queries per sequence at absolute positions q_pos0 + t,
    N cached keys per sequence.  Indexer: H_I heads of width D_I.  Top-k:
    K = index_topk.  Sparse MLA: H heads over D-wide latent rows whose first
    DV entries are the value.  ``stages`` names the steps the workload runs.
    """
    name: str
    wid: int
    dtype: str
    B: int
    Tq: int
    N: int
    q_pos0: int
    H_I: int
    D_I: int
    K: int
    H: int
    D: int
    DV: int
    scale: float
    stages: tuple
    dists: dict = field(default_factory=dict)

    def shape(self, name: str) -> tuple:
        return {
            "q_idx": (self.B, self.Tq, self.H_I, self.D_I),
            "k_idx": (self.B, self.N, self.D_I),
            "w": (self.B, self.Tq, self.H_I),
            "q": (self.B, self.Tq, self.H, self.D),
            "kv": (self.B, self.N, self.D),
            "idx": (self.B, self.Tq, self.K),
        }[name]

    def inputs(self) -> tuple:
        names = []
        if "index" in self.stages:
            names += ["q_idx", "k_idx", "w"]
        if "mla" in self.stages:
            names += ["q", "kv"]
            if "topk" not in self.stages:
                names += ["idx"]
        return tuple(names)

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


INT3 = Dist("int", -3, 3)
INT4 = Dist("int", -4, 4)
NORMAL = Dist("normal")
POW2_M4_0 = Dist("pow2", -4, 0)
W_SET = Dist("choice", values=(0.25, 0.5, 1.0, 2.0))

WORKLOADS = {
    # L=256 causal prefill in fp32; indexer 4x32, top-32; MLA 4 heads, 64+16 wide
    "tiny_prefill_f32": Workload(
        "tiny_prefill_f32", 1, "f32", B=1, Tq=256, N=256, q_pos0=0, H_I=4, D_I=32, K=32,
        H=4, D=80, DV=64, scale=1.0 / math.sqrt(80.0), stages=("index", "topk", "mla"),
        dists={"q_idx": INT3, "k_idx": INT3, "w": W_SET, "q": NORMAL, "kv": NORMAL}),
    # L=8192 causal prefill, indexer 64x128 + top-2048 only
    "indexer_topk_prefill_8k": Workload(
        "indexer_topk_prefill_8k", 2, "bf16", B=1, Tq=8192, N=8192, q_pos0=0, H_I=64, D_I=128,
        K=2048, H=128, D=576, DV=512, scale=1.0 / math.sqrt(192.0), stages=("index", "topk"),
        dists={"q_idx": INT4, "k_idx": INT4, "w": POW2_M4_0}),
    # batch-64 decode over a 32768-row latent cache, 2048 given indices per query
    "sparse_mla_decode_b64_32k": Workload(
        "sparse_mla_decode_b64_32k", 3, "bf16", B=64, Tq=1, N=32768, q_pos0=32767, H_I=64,
        D_I=128, K=2048, H=128, D=576, DV=512, scale=1.0 / math.sqrt(192.0), stages=("mla",),
        dists={"q": NORMAL, "kv": NORMAL}),
    # L=16384 full causal prefill: indexer -> top-2048 -> sparse MLA
    "dsa_prefill_16k": Workload(
        "dsa_prefill_16k", 4, "bf16", B=1, Tq=16384, N=16384, q_pos0=0, H_I=64, D_I=128, K=2048,
        H=128, D=576, DV=512, scale=1.0 / math.sqrt(192.0), stages=("index", "topk", "mla"),
        dists={"q_idx": INT3, "k_idx": INT3, "w": W_SET, "q": NORMAL, "kv": NORMAL}),
    # batch-32 decode at 131072 context: indexer over all keys -> top-2048 -> sparse MLA
    "dsa_decode_b32_128k": Workload(
        "dsa_decode_b32_128k", 5, "bf16", B=32, Tq=1, N=131072, q_pos0=131071, H_I=64, D_I=128,
        K=2048, H=128, D=576, DV=512, scale=1.0 / math.sqrt(192.0), stages=("index", "topk", "mla"),
        dists={"q_idx": INT4, "k_idx": INT4, "w": POW2_M4_0, "q": NORMAL, "kv": NORMAL}),
}


def tensor_flat(wl: Workload, name: str, start: int, count: int, seed: int = 0) -> np.ndarray:
    """Flat elements [start, start+count) of tensor `name` of workload `wl`."""
    key = stream_key(seed, wl.wid, TENSOR_IDS[name])
    return fill(key, start, count, wl.dists[name], wl.dtype)


def tensor(wl: Workload, name: str, seed: int = 0) -> np.ndarray:
    """The whole tensor `name`, shaped."""
    shp = wl.shape(name)
    if name == "idx":
        key = stream_key(seed, wl.wid, TENSOR_IDS["idx"])
        return floyd(key, wl.B * wl.Tq, wl.N, wl.K).reshape(shp)
    return tensor_flat(wl, name, 0, int(np.prod(shp)), seed).reshape(shp)


def rows(wl: Workload, name: str, b: int, row_ids, seed: int = 0) -> np.ndarray:
    """Rows `row_ids` (second axis) of sequence b of a [B, R, ...] tensor."""
    shp = wl.shape(name)
    width = int(np.prod(shp[2:]))
    out = []
    for r in np.asarray(row_ids, dtype=np.int64).reshape(-1):
        start = (b * shp[1] + int(r)) * width
        out.append(tensor_flat(wl, name, start, width, seed))
    return np.stack(out).reshape((len(out),) + shp[2:]) if out else np.empty((0,) + shp[2:])


def row_block(wl: Workload, name: str, b: int, r0: int, r1: int, seed: int = 0) -> np.ndarray:
    """Contiguous rows [r0, r1) of sequence b of a [B, R, ...] tensor."""
    shp = wl.shape(name)
    width = int(np.prod(shp[2:]))
    start = (b * shp[1] + r0) * width
    return tensor_flat(wl, name, start, (r1 - r0) * width, seed).reshape((r1 - r0,) + shp[2:])


def make_inputs(wl: Workload, seed: int = 0) -> dict:
    return {n: tensor(wl, n, seed) for n in wl.inputs()}
