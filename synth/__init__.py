"""Seeded synthetic inputs for the LongCat Sparse Attention (LSA) hot path.

This module only draws random numbers and stores them in the cache formats the
path consumes (bf16 bit patterns, OCP fp8-e4m3fn bytes with a per-token fp32
scale).  It holds none of the method's arithmetic: no scores, no selection, no
attention.  Both the CPU oracle and the GPU path read the same arrays produced
here.

The five workloads follow the statement of the problem on the LongCat pages
(LongCat-Flash-Lite-Sparse summary, "technical features": a sink plus a local
window plus a top-k fill; hierarchical block pre-selection; cross-layer reuse)
with the shapes, dtypes and value distributions of the benchmark configurations:

  c1  tiny decode      B=1, N=4096, T=8, indexer 4x64 bf16, MQA 16 heads d=128,
                       K=512, sink 16, window 128, 32 salient keys
  c2  128K MLA decode  B=8, N=131072, T=1, indexer 64x128 fp8+scale, MLA 64 heads
                       row 576 (V = first 512), K=2048, sink 64, window 512,
                       1% salient keys
  c3  1M HI decode     B=1, N=1048576, T=4, indexer 4x64 bf16, MQA 16 heads,
                       blocks of 64, keep 256, K=2048/64/512, 40 salient blocks
  c4  chunked prefill  B=1, N=262144+4096, T=4096, indexer 64x128 fp8, GQA 64/8,
                       K=2048/64/512
  c5  4-layer CLI      B=16, N=65536, T=1, indexer 32x128 fp8, per layer GQA 32/4

Distributions (readings where the statement is silent are marked R):
  q, k, v, indexer q/k ~ N(0,1)/sqrt(d) of the tensor's last dim; MLA rows ~ N(0,1);
  indexer weights w ~ U(0,1) (R for c2..c5); salient keys have their indexer key
  multiplied by 4 before quantisation (R: the c1 definition, reused for c2/c3).
  fp8 keys: scale = max(amax_row, 1e-12)/448 in fp32, bytes = e4m3fn(clamp(k/scale,
  +-448)) with round-to-nearest-even (torch's cast).
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import hashlib
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = ["LSAConfig", "CONFIGS", "config", "make_inputs", "to_bf16_bits", "to_e4m3fn",
           "digest"]


@dataclass(frozen=True)
class LSAConfig:
    name: str
    cid: int
    B: int
    T: int
    N: int                  # cache rows per sequence (the T queries are the last T rows)
    H_I: int                # indexer heads
    D_I: int                # indexer dim
    k_fp8: bool             # indexer keys stored as fp8-e4m3fn + per-token fp32 scale
    Hq: int
    Hkv: int
    d_qk: int
    d_v: int
    mla: bool               # one shared latent row per token; V = its first d_v columns
    K: int                  # total budget per query token (sink + window + fill)
    S: int                  # sink
    W: int                  # local window (ends at the query position, inclusive)
    hi: bool = False        # hierarchical (block) pre-selection
    q_fp8: bool = False     # indexer queries quantised to fp8 per (token, head) row
    Bs: int = 64            # HI block size
    n_keep: int = 256       # HI kept blocks per query token
    layers: int = 1         # consecutive layers sharing one selection (CLI)
    salient: str = "none"   # "keys:<count>", "frac:<fraction>", "blocks:<count>", "none"

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def tau(self) -> float:
        return float(1.0 / np.sqrt(self.d_qk))

    def scaled(self, **kw) -> "LSAConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    1: LSAConfig("c1_tiny_decode", 1, B=1, T=8, N=4096, H_I=4, D_I=64, k_fp8=False,
                 Hq=16, Hkv=1, d_qk=128, d_v=128, mla=False, K=512, S=16, W=128,
                 salient="keys:32"),
    2: LSAConfig("c2_mla_decode_128k", 2, B=8, T=1, N=131072, H_I=64, D_I=128, k_fp8=True,
                 Hq=64, Hkv=1, d_qk=576, d_v=512, mla=True, K=2048, S=64, W=512,
                 salient="frac:0.01"),
    3: LSAConfig("c3_hi_decode_1m", 3, B=1, T=4, N=1048576, H_I=4, D_I=64, k_fp8=False,
                 Hq=16, Hkv=1, d_qk=128, d_v=128, mla=False, K=2048, S=64, W=512,
                 hi=True, Bs=64, n_keep=256, salient="blocks:40"),
    4: LSAConfig("c4_chunked_prefill_256k", 4, B=1, T=4096, N=262144 + 4096, H_I=64, D_I=128,
                 k_fp8=True, Hq=64, Hkv=8, d_qk=128, d_v=128, mla=False, K=2048, S=64, W=512),
    5: LSAConfig("c5_cli_decode_64k", 5, B=16, T=1, N=65536, H_I=32, D_I=128, k_fp8=True,
                 Hq=32, Hkv=4, d_qk=128, d_v=128, mla=False, K=2048, S=64, W=512, layers=4),
}


def config(cid: int, **overrides) -> LSAConfig:
    c = CONFIGS[cid]
    return c.scaled(**overrides) if overrides else c


# ----------------------------------------------------------------------------- casts

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (torch's cast,
    used here only as a format converter on the CPU)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3fn(x: np.ndarray):
    """Per-row fp8 storage of a [..., D] float32 array.

    Returns (bytes uint8 [..., D], scale float32 [...]).  scale = max(amax, 1e-12)/448
    computed in fp32; bytes = e4m3fn(clamp(x/scale, +-448)) rounded to nearest even by
    torch's cast (torch is used here only as a format converter on the CPU).
    """
    import torch
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    amax = xt.abs().amax(dim=-1)
    scale = torch.clamp(amax, min=1e-12) / 448.0
    y = torch.clamp(xt / scale.unsqueeze(-1), -448.0, 448.0)
    b = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return b, scale.numpy().astype(np.float32)


# ----------------------------------------------------------------------------- draws

_CHUNK = 1 << 22


def _normal(ss: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    """N(0, std^2) float32.  Chunk i of 2^22 values is drawn from its own PCG64 stream
    (the i-th child of `ss`), so the values do not depend on how many threads fill them."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    kids = ss.spawn((n + _CHUNK - 1) // _CHUNK)

    def fill(i):
        s, e = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        np.random.Generator(np.random.PCG64(kids[i])).standard_normal(e - s, dtype=np.float32, out=out[s:e])

    workers = min(len(kids), 16, os.cpu_count() or 1)
    if workers > 1:
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(len(kids))))
    else:
        for i in range(len(kids)):
            fill(i)
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def _salient_positions(rng, cfg: LSAConfig, b: int):
    """Positions whose indexer key is planted x4 (never inside a forced sink/window)."""
    kind, _, arg = cfg.salient.partition(":")
    p0 = cfg.N - cfg.T                      # first query position
    lo, hi = cfg.S, max(cfg.S, p0 - cfg.W + 1)
    if kind == "none" or hi <= lo:
        return np.zeros(0, dtype=np.int64)
    if kind == "keys":
        cnt = min(int(arg), hi - lo)
        return np.sort(rng.choice(np.arange(lo, hi), size=cnt, replace=False))
    if kind == "frac":
        cnt = min(int(round(float(arg) * cfg.N)), hi - lo)
        return np.sort(rng.choice(np.arange(lo, hi), size=cnt, replace=False))
    if kind == "blocks":
        nb = cfg.N // cfg.Bs
        last = max(2, nb - 10)
        cnt = min(int(arg), last - 1)
        blocks = np.sort(rng.choice(np.arange(1, last), size=cnt, replace=False))
        return (blocks[:, None] * cfg.Bs + np.arange(cfg.Bs)[None, :]).reshape(-1)
    raise ValueError(cfg.salient)


def make_inputs(cfg: LSAConfig, seed: Optional[int] = None, with_kv: bool = True) -> dict:
    """Draw every input of one workload.

    Child streams of SeedSequence(seed) are used in a fixed order:
    qI, w, kI, salient, then per layer (q, k, v).  Returned arrays hold raw storage:
      qI  uint16 bf16 bits [B,T,H_I,D_I]      w  float32 [B,T,H_I]
      kI  uint16 bf16 bits or uint8 e4m3fn [B,N,D_I];  kI_scale float32 [B,N] or None
      q   uint16 [L,B,T,Hq,d_qk]
      k   uint16 [L,B,N,Hkv,d_qk] (MLA: [L,B,N,1,576], v is None and V = k[..., :d_v])
      v   uint16 [L,B,N,Hkv,d_v] or None
      ctx_len int32 [B] (= N), salient list of int64 arrays (one per sequence)
    """
    seed = 1000 + cfg.cid if seed is None else seed
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(4 + 3 * cfg.layers)
    sq, sw, sk, ssal = kids[:4]
    rw = np.random.Generator(np.random.PCG64(sw))
    rs = np.random.Generator(np.random.PCG64(ssal))
    B, T, N = cfg.B, cfg.T, cfg.N
    out = {"cfg": cfg, "seed": seed}
    qI = _normal(sq, (B, T, cfg.H_I, cfg.D_I), 1.0 / np.sqrt(cfg.D_I))
    out["qI"] = to_bf16_bits(qI)
    out["w"] = rw.random((B, T, cfg.H_I), dtype=np.float32)
    kI = _normal(sk, (B, N, cfg.D_I), 1.0 / np.sqrt(cfg.D_I))
    sal = []
    for b in range(B):
        pos = _salient_positions(rs, cfg, b)
        kI[b, pos, :] *= np.float32(4.0)
        sal.append(pos)
    out["salient"] = sal
    if cfg.k_fp8:
        out["kI"], out["kI_scale"] = to_e4m3fn(kI)
    else:
        out["kI"], out["kI_scale"] = to_bf16_bits(kI), None
    del kI
    out["ctx_len"] = np.full(B, N, dtype=np.int32)
    if with_kv:
        qs, ks, vs = [], [], []
        for layer in range(cfg.layers):
            r_q, r_k, r_v = kids[4 + 3 * layer: 7 + 3 * layer]
            if cfg.mla:
                qs.append(to_bf16_bits(_normal(r_q, (B, T, cfg.Hq, cfg.d_qk), 1.0 / np.sqrt(cfg.d_qk))))
                ks.append(to_bf16_bits(_normal(r_k, (B, N, 1, cfg.d_qk), 1.0)))
            else:
                qs.append(to_bf16_bits(_normal(r_q, (B, T, cfg.Hq, cfg.d_qk), 1.0 / np.sqrt(cfg.d_qk))))
                ks.append(to_bf16_bits(_normal(r_k, (B, N, cfg.Hkv, cfg.d_qk), 1.0 / np.sqrt(cfg.d_qk))))
                vs.append(to_bf16_bits(_normal(r_v, (B, N, cfg.Hkv, cfg.d_v), 1.0 / np.sqrt(cfg.d_v))))
        out["q"] = np.stack(qs)
        out["k"] = np.stack(ks)
        out["v"] = np.stack(vs) if vs else None
    return out


def digest(inputs: dict) -> str:
    """sha256 over every array of a draw, in a fixed key order (logged by tests/bench)."""
    h = hashlib.sha256()
    for key in ("qI", "w", "kI", "kI_scale", "q", "k", "v", "ctx_len"):
        a = inputs.get(key)
        if a is not None:
            h.update(key.encode())
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
