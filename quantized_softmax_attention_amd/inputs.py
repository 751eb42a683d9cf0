"""Seeded synthetic inputs for the attention forward.

This module holds none of the method's arithmetic: it only draws random numbers
and lays them out.  Both the HIP path (tests, benchmark) and the CPU oracle are
fed from here, so they always see the same bf16 bits.

The benchmark artefacts this library follows measured real block-24 activations
of a video diffusion transformer ("gb10-sage2-p0-interleave-softmax-latency.json",
metadata: 1344x768, 124 frames, block_index 24; q_shape [1, 37810, 56, 128]).
Those activations need the trained model, so seeded stand-ins of the same shapes
and layouts are drawn instead:

* ``hnd_case``    -- Q, K, V ~ N(0, 1) as contiguous [B, H, N, D] (HND) tensors;
                     K gets a per-(b, h, d) offset ~ N(0, 2) shared by all tokens.
* ``packed_case`` -- one bf16 buffer X [B, N, 3*H*D] ~ N(0, 1), the packed output
                     of the QKV projection (strided page, "dataflow.qkv_input":
                     projection-strided NHD views, no materialisation).  Q, K, V
                     are the column ranges [0, HD), [HD, 2HD), [2HD, 3HD) viewed
                     as [B, N, H, D] with row stride 3*H*D; K gets the offset.
                     ``stress=True``: per (b, h), 4 distinct channels of Q and K
                     are scaled x10 (before the K offset) and V is Student-t with
                     3 degrees of freedom.

Random numbers come from torch CPU generators, one per (seed, stream, row chunk)
so that generation can run on several threads and stays reproducible.  Values
are drawn in fp32 and rounded once to bf16 (round to nearest even).
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

# stream ids: each random component has its own stream
(_S_Q, _S_K, _S_V, _S_OFFSET, _S_OUTLIER, _S_T_NUM, _S_T_DEN, _S_ROWS, _S_X, _S_MX_EXP, _S_MX_KIND,
 _S_GAMMA) = range(1, 13)
_CHUNK_ROWS = 512


def _seed(seed: int, stream: int, chunk: int) -> int:
    h = hashlib.sha256(f"{seed}:{stream}:{chunk}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, stream: int, chunk: int = 0) -> torch.Generator:
    return torch.Generator().manual_seed(_seed(seed, stream, chunk))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(rows: int, fn):
    """Call fn(chunk_index, r0, r1) for fixed row chunks, on a thread pool."""
    nchunks = -(-rows // _CHUNK_ROWS)
    spans = [(c, c * _CHUNK_ROWS, min(rows, (c + 1) * _CHUNK_ROWS)) for c in range(nchunks)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda s: fn(*s), spans))


def normal_f32(shape, seed: int, stream: int, std: float = 1.0) -> torch.Tensor:
    """N(0, std^2) in fp32, drawn in row chunks of the flattened leading dims."""
    shape = tuple(shape)
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    cols = shape[-1]
    out = torch.empty(rows, cols, dtype=torch.float32)

    def fill(c, r0, r1):
        out[r0:r1] = torch.randn(r1 - r0, cols, generator=_gen(seed, stream, c)) * std

    _chunked(rows, fill)
    return out.reshape(shape)


def student_t3_f32(shape, seed: int) -> torch.Tensor:
    """Student-t, 3 degrees of freedom: Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3)."""
    z = normal_f32(shape, seed, _S_T_NUM)
    chi = normal_f32(tuple(shape) + (3,), seed, _S_T_DEN)
    return z / torch.sqrt((chi * chi).sum(-1) / 3.0)


@dataclass
class Case:
    """One workload: bf16 CPU tensors plus [B, N, H, D] views of Q, K, V."""
    name: str
    B: int
    N: int
    H: int
    D: int
    q: torch.Tensor            # [B, N, H, D] views (possibly strided) of bf16 CPU storage
    k: torch.Tensor
    v: torch.Tensor
    packed: torch.Tensor | None = None   # the [B, N, 3HD] buffer for packed cases

    def to(self, device) -> "Case":
        """Copy to `device` preserving the layout (packed views stay views)."""
        if self.packed is not None:
            p = self.packed.to(device)
            HD = self.H * self.D
            q, k, v = (p[:, :, i * HD:(i + 1) * HD].unflatten(2, (self.H, self.D)) for i in range(3))
            return Case(self.name, self.B, self.N, self.H, self.D, q, k, v, p)
        return Case(self.name, self.B, self.N, self.H, self.D,
                    *(t.transpose(1, 2).contiguous().to(device).transpose(1, 2)
                      for t in (self.q, self.k, self.v)))


def hnd_case(B: int, N: int, H: int, D: int = 128, seed: int = 0, name: str = "hnd") -> Case:
    """Contiguous HND Q/K/V ~ N(0, 1); K += offset[b, h, d] ~ N(0, 2)."""
    q = normal_f32((B, H, N, D), seed, _S_Q)
    k = normal_f32((B, H, N, D), seed, _S_K)
    v = normal_f32((B, H, N, D), seed, _S_V)
    off = normal_f32((B, H, 1, D), seed, _S_OFFSET, std=2.0)
    k = k + off
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    # [B, H, N, D] storage viewed as [B, N, H, D]
    return Case(name, B, N, H, D, q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2))


def outlier_channels(B: int, H: int, D: int, seed: int, count: int = 4) -> torch.Tensor:
    """Per (b, h): `count` distinct channel indices, [B, H, count] int64."""
    g = _gen(seed, _S_OUTLIER)
    return torch.stack([torch.randperm(D, generator=g)[:count] for _ in range(B * H)]).reshape(B, H, count)


def packed_case(B: int, N: int, H: int, D: int = 128, seed: int = 0, stress: bool = False,
                name: str = "packed") -> Case:
    """Packed QKV projection buffer X [B, N, 3HD] bf16 with strided Q/K/V views."""
    HD = H * D
    C = 3 * HD
    off = normal_f32((B, 1, H, D), seed, _S_OFFSET, std=2.0).reshape(B, 1, HD)
    scale = torch.ones(B, 1, H, D)
    if stress:
        idx = outlier_channels(B, H, D, seed)
        scale.scatter_(3, idx.unsqueeze(1), 10.0)
    scale = scale.reshape(B, 1, HD)
    X = torch.empty(B * N, C, dtype=torch.bfloat16)
    rows = B * N

    def fill(c, r0, r1):
        x = torch.randn(r1 - r0, C, generator=_gen(seed, _S_X, c))
        b = torch.arange(r0, r1) // N
        if stress:
            x[:, :HD] *= scale[b, 0]
            x[:, HD:2 * HD] *= scale[b, 0]
        x[:, HD:2 * HD] += off[b, 0]
        if stress:
            z = torch.randn(r1 - r0, HD, generator=_gen(seed, _S_T_NUM, c))
            chi = torch.randn(r1 - r0, HD, 3, generator=_gen(seed, _S_T_DEN, c))
            x[:, 2 * HD:] = z / torch.sqrt((chi * chi).sum(-1) / 3.0)
        X[r0:r1] = x.to(torch.bfloat16)

    _chunked(rows, fill)
    X = X.reshape(B, N, C)
    q, k, v = (X[:, :, i * HD:(i + 1) * HD].unflatten(2, (H, D)) for i in range(3))
    return Case(name, B, N, H, D, q, k, v, X)


def sample_rows(B: int, H: int, N: int, count: int = 512, tail: int = 64, seed: int = 0) -> np.ndarray:
    """Query rows checked at full size, [B, H, R] int32, sorted per (b, h).

    Per (b, h): the last `tail` rows (they cover a ragged last tile) plus
    count - tail distinct rows drawn from [0, N - tail).  All rows if N <= count.
    """
    if N <= count:
        return np.broadcast_to(np.arange(N, dtype=np.int32), (B, H, N)).copy()
    g = _gen(seed, _S_ROWS)
    out = np.empty((B, H, count), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            pick = torch.randperm(N - tail, generator=g)[:count - tail].numpy()
            rows = np.concatenate([np.sort(pick), np.arange(N - tail, N)])
            out[b, h] = rows.astype(np.int32)
    return out


# The five workloads: tiny (N=256, H=2), mid (N=4096, H=56), block-24 packed
# (N=37810, H=56), the same through the bf16 path, and the two-sequence stress.
# name -> (B, N, H, D, layout, stress)
CONFIGS = {
    "tiny": (1, 256, 2, 128, "hnd", False),
    "mid": (1, 4096, 56, 128, "hnd", False),
    "block24": (1, 37810, 56, 128, "packed", False),
    "block24_bf16": (1, 37810, 56, 128, "packed", False),
    "stress": (2, 37810, 56, 128, "packed", True),
}


def config(name: str, seed: int = 0) -> Case:
    B, N, H, D, layout, stress = CONFIGS[name]
    if layout == "hnd":
        return hnd_case(B, N, H, D, seed=seed, name=name)
    return packed_case(B, N, H, D, seed=seed, stress=stress, name=name)


def mx_tensor(B: int, N: int, H: int, D: int = 128, seed: int = 0) -> torch.Tensor:
    """A contiguous bf16 [B, N, H, D] tensor for microscaling tests: N(0, 1) values,
    each 32-channel block scaled by 2^e with e uniform in [-60, 60], and blocks
    picked at random (about 1 in 16 of each kind) set to zero, to -0.0, to one
    nonzero value among zeros, or to values near the bottom of the bf16 range
    (2^-140 .. 2^-120, subnormals included)."""
    x = normal_f32((B, N, H, D), seed, _S_X)
    nb = B * N * H * (D // 32)
    g = _gen(seed, _S_MX_EXP)
    e = torch.randint(-60, 61, (nb, 1), generator=g).float()
    kind = torch.randint(0, 16, (nb,), generator=_gen(seed, _S_MX_KIND))
    blocks = x.reshape(nb, 32) * torch.exp2(e)
    blocks[kind == 0] = 0.0
    blocks[kind == 1] = -0.0
    lone = kind == 2
    blocks[lone, 1:] = 0.0
    tiny = kind == 3
    blocks[tiny] = x.reshape(nb, 32)[tiny] * torch.exp2(torch.randint(-140, -119, (int(tiny.sum()), 1), generator=g).float())
    return blocks.reshape(B, N, H, D).to(torch.bfloat16)


@dataclass
class NormRope:
    """Parameters of the RMSNorm + RoPE applied to Q and K before quantisation."""
    gamma_q: torch.Tensor     # [D] fp32 (bf16-representable values)
    gamma_k: torch.Tensor     # [D] fp32
    rope: torch.Tensor        # [N, D/2, 2] fp32: (cos, sin) of each token's angle per channel pair
    eps: float

    def to(self, device) -> "NormRope":
        return NormRope(self.gamma_q.to(device), self.gamma_k.to(device), self.rope.to(device), self.eps)


def video_rope_table(N: int, D: int = 128, width: int = 42, height: int = 24, theta: float = 10000.0) -> torch.Tensor:
    """Rotary angles of a video token grid: token n sits at frame n // (w*h), row
    and column of a width x height latent frame (1344x768 with 32-pixel cells);
    the D/2 channel pairs split into frame / row / column bands of 16 / 24 / 24
    pairs, band pair j at frequency theta^(-j / band).  cos and sin are computed
    in fp64 and rounded to fp32.  [N, D/2, 2]"""
    pairs = D // 2
    bands = [pairs // 4, (pairs - pairs // 4) // 2]
    bands.append(pairs - bands[0] - bands[1])
    n = np.arange(N, dtype=np.int64)
    pos = [n // (width * height), (n // width) % height, n % width]
    ang = np.empty((N, pairs), np.float64)
    p0 = 0
    for band, ps in zip(bands, pos):
        freq = theta ** (-np.arange(band, dtype=np.float64) / band)
        ang[:, p0:p0 + band] = ps[:, None].astype(np.float64) * freq[None, :]
        p0 += band
    tab = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    return torch.from_numpy(tab)


def norm_rope_params(N: int, D: int = 128, seed: int = 0, eps: float = 1e-6) -> NormRope:
    """Seeded RMSNorm weights (uniform in [0.5, 1.5), rounded to bf16 values) for
    Q and K, the video rotary table and eps."""
    g = _gen(seed, _S_GAMMA)
    gq = (0.5 + torch.rand(D, generator=g)).to(torch.bfloat16).float()
    gk = (0.5 + torch.rand(D, generator=g)).to(torch.bfloat16).float()
    return NormRope(gq, gk, video_rope_table(N, D), eps)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a contiguous bf16 CPU tensor (no copy)."""
    assert t.dtype == torch.bfloat16 and t.is_contiguous() and t.device.type == "cpu"
    return t.view(torch.int16).numpy().view(np.uint16)
