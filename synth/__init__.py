"""Seeded synthetic workloads for the sparse-MQA decode path.

This module only draws random numbers and *encodes* them into the storage
formats the path reads: OCP FP8 E4M3 bytes, OCP MX E2M1 nibbles with E8M0
block exponents (plus an optional fp32 row scale), bf16 queries, int32/int64
layout arrays.  It holds none of the path's arithmetic: no decoding, scoring,
selection or attention.  Both the CPU oracle (``oracle/``) and the GPU library
consume what it produces; neither is imported here.

Workloads (sizes from the method's setting: an FP4 global latent of ~890 B per
token shared by every head, an FP8 128-position sliding window, an FP8
multi-head indexer, top-k selection; bounded replay re-runs the last 128
tokens of a prefix hit with the window clipped at s = H - 128):

  tiny          1 query, n=4096, indexer 8x64, k=256, attention 16x512, no row scale
  decode_8k     1 query, n=8192, indexer 64x128, k=2048, attention 64x1664, row scale
  ragged_b32    32 queries, n_b ~ U[16384, 65536], otherwise as decode_8k
  decode_512k   4 queries, n=524288, 1% of indexer keys offset by +3 (peaked scores)
  replay_h100k  8 sessions x 128 replay queries, prefix H=100000, window clipped at H-128

Random recipe: ``numpy.random.SeedSequence(seed).spawn(8)`` gives one child per
stream, in this order: 0 indexer q, 1 head weights, 2 indexer keys,
3 attention q, 4 global latent, 5 window rows, 6 lengths and candidate sets,
7 peak positions.  Children 0-5 seed a ``torch.Generator`` on the target device
(so data drawn on CPU and on GPU differ for one seed; each is reproducible),
drawn in row-major chunks of 65536 rows.  Children 6-7 drive numpy PCG64.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

CHUNK_ROWS = 65536

# Workload definitions.  ``lengths`` is either an int (every sequence) or a
# (lo, hi) range drawn per sequence; ``replay`` is (H, queries per session).
WORKLOADS = {
    "tiny": dict(B=1, lengths=4096, Hi=8, Di=64, k=256, Hq=16, D=512, W=128,
                 rowscale=False, peak_frac=0.0, replay=None),
    "decode_8k": dict(B=1, lengths=8192, Hi=64, Di=128, k=2048, Hq=64, D=1664, W=128,
                      rowscale=True, peak_frac=0.0, replay=None),
    "ragged_b32": dict(B=32, lengths=(16384, 65536), Hi=64, Di=128, k=2048, Hq=64, D=1664,
                       W=128, rowscale=True, peak_frac=0.0, replay=None),
    "decode_512k": dict(B=4, lengths=524288, Hi=64, Di=128, k=2048, Hq=64, D=1664, W=128,
                        rowscale=True, peak_frac=0.01, replay=None),
    "replay_h100k": dict(B=8, lengths=100000, Hi=64, Di=128, k=2048, Hq=64, D=1664, W=128,
                         rowscale=True, peak_frac=0.0, replay=(100000, 128)),
}

N_CAND_DEFAULT = 16384


@dataclass
class Workload:
    """One batch of inputs, in the exact byte layouts the library takes."""
    name: str
    B: int
    T: int
    Hi: int
    Di: int
    k: int
    Hq: int
    D: int
    W: int
    sm_scale: float
    max_ctx: int                     # max over queries of the scored-set size
    seq_start: torch.Tensor          # int64 [B+1]
    q_start: torch.Tensor            # int32 [B+1]  queries of seq b: [q_start[b], q_start[b+1])
    q_pos: torch.Tensor              # int32 [T]    absolute position of each query (inclusive bound)
    qI: torch.Tensor                 # uint8 [T, Hi, Di]   E4M3 indexer queries
    w: torch.Tensor                  # float32 [T, Hi]     indexer head weights
    kI: torch.Tensor                 # uint8 [N, Di]       E4M3 indexer keys
    kscale: Optional[torch.Tensor]   # float32 [N] or None
    q: torch.Tensor                  # bfloat16 [T, Hq, D] attention queries
    kv_codes: torch.Tensor           # uint8 [N, D/2]      E2M1, low nibble = even element
    kv_e8m0: torch.Tensor            # uint8 [N, D/32]     E8M0 block exponents
    kv_rowscale: Optional[torch.Tensor]  # float32 [N] or None
    swa: torch.Tensor                # uint8 [B, W, D]     E4M3 window rows
    swa_scale: Optional[torch.Tensor]    # float32 [B, W] or None
    swa_pos0: torch.Tensor           # int32 [B]           position of window row 0
    swa_clip: Optional[torch.Tensor]     # int32 [T] or None   clip start s_t
    cand: Optional[torch.Tensor] = None  # int32 [T, n_cand]   ascending candidate positions
    kv_fp8: Optional[torch.Tensor] = None        # uint8 [N, D]  E4M3 global latent (FP8 cache)
    kv_fp8_scale: Optional[torch.Tensor] = None  # float32 [N]   its row scales
    kv_nv_codes: Optional[torch.Tensor] = None   # uint8 [N, D/2]  NVFP4 global latent: E2M1
    kv_nv_scales: Optional[torch.Tensor] = None  # uint8 [N, D/16] E4M3 scale per 16 elements
    kv_nv_global: float = 1.0                    # its fp32 tensor scale
    meta: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return int(self.kI.shape[0])

    def to(self, device) -> "Workload":
        out = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            out[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Workload(**out)

    def cpu(self) -> "Workload":
        return self.to("cpu")


# ----------------------------------------------------------------------------
# Encoders (input preparation only)
# ----------------------------------------------------------------------------

def encode_e4m3(x: torch.Tensor) -> torch.Tensor:
    """float32 -> OCP E4M3FN bytes: saturate to +-448, then round to nearest even."""
    return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _e2m1_round(y: torch.Tensor) -> torch.Tensor:
    """float32 -> 4-bit E2M1 codes (bit 3 = sign), round-to-nearest-even, saturating at 6."""
    grid = torch.tensor(_E2M1_GRID, dtype=torch.float32, device=y.device)
    a = y.abs()
    lo = (torch.bucketize(a, grid, right=True) - 1).clamp(0, 7)
    hi = (lo + 1).clamp(max=7)
    glo, ghi = grid[lo], grid[hi]
    mid = (glo + ghi) * 0.5
    up = (a > mid) | ((a == mid) & (lo % 2 == 1))
    mag = torch.where(up & (hi != lo), hi, lo)
    mag = torch.where(a >= 6.0, torch.full_like(mag, 7), mag)
    sign = ((y < 0) & (mag > 0)).to(torch.int64) << 3
    return (mag | sign).to(torch.uint8)


def encode_mx_e2m1(x: torch.Tensor, rowscale: bool):
    """float32 rows [R, D] -> (codes uint8 [R, D/2], e8m0 uint8 [R, D/32], rho float32 [R] | None).

    With ``rowscale`` the row is first divided by rho = amax|row| / 6 (1 for a
    zero row).  Each 32-element block then gets the OCP MX shared exponent
    E = floor(log2(block amax)) - 2 + 127 (clamped to [0, 254], 0 for an
    all-zero block) and its elements are rounded to E2M1 after division by
    2^(E-127).  Element 2i goes to the low nibble of byte i.
    """
    R, D = x.shape
    assert D % 32 == 0
    if rowscale:
        amax = x.abs().amax(dim=1)
        rho = torch.where(amax > 0, amax / 6.0, torch.ones_like(amax))
        xs = x / rho[:, None]
    else:
        rho = None
        xs = x
    blocks = xs.view(R, D // 32, 32)
    bmax = blocks.abs().amax(dim=2)
    _, ex = torch.frexp(bmax)                  # bmax = m * 2^ex, m in [0.5, 1)
    E = (ex.to(torch.int32) - 1 - 2 + 127).clamp(0, 254)
    E = torch.where(bmax > 0, E, torch.zeros_like(E))
    scale = torch.ldexp(torch.ones_like(bmax), (E - 127).to(torch.float32))
    y = blocks / scale[..., None]
    codes = _e2m1_round(y).view(R, D).to(torch.int32)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).to(torch.uint8)
    return packed, E.to(torch.uint8), rho


# ----------------------------------------------------------------------------
# Generator
# ----------------------------------------------------------------------------

def _children(seed: int):
    return np.random.SeedSequence(seed).spawn(8)


def _torch_gen(child, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(child.generate_state(1, dtype=np.uint32)[0]))
    return g


def _randn_rows(g, rows, cols, device, fn):
    """Draw N(0,1) float32 [rows, cols] in chunks of CHUNK_ROWS rows and hand each to fn(r0, block)."""
    for r0 in range(0, rows, CHUNK_ROWS):
        r = min(CHUNK_ROWS, rows - r0)
        fn(r0, torch.randn((r, cols), generator=g, device=device, dtype=torch.float32))


def workload_params(name: str, **overrides) -> dict:
    p = dict(WORKLOADS[name])
    p.update(overrides)
    return p


def generate(name: str, seed: int = 0, device="cpu", n_cand: Optional[int] = None,
             **overrides) -> Workload:
    """Build the named workload (optionally resized by ``overrides``) on ``device``.

    ``n_cand`` switches on candidate mode: each query gets ``n_cand`` sorted
    positions drawn without replacement from its sequence (padded with
    positions past the query when the sequence is shorter).
    """
    p = workload_params(name, **overrides)
    B, Hi, Di, k, Hq, D, W = (p[x] for x in ("B", "Hi", "Di", "k", "Hq", "D", "W"))
    ch = _children(seed)
    rng_len = np.random.Generator(np.random.PCG64(ch[6]))
    rng_peak = np.random.Generator(np.random.PCG64(ch[7]))

    # ---- layout ----
    if p["replay"] is not None:
        H, nq = p["replay"]
        lengths = np.full(B, H, dtype=np.int64)
        q_counts = np.full(B, nq, dtype=np.int64)
        q_pos = np.concatenate([H - nq + np.arange(nq) for _ in range(B)]).astype(np.int32)
        swa_pos0 = np.full(B, H - W, dtype=np.int32)
        swa_clip = np.full(int(q_counts.sum()), H - nq, dtype=np.int32)
    else:
        L = p["lengths"]
        if isinstance(L, (tuple, list)):
            lengths = rng_len.integers(L[0], L[1], endpoint=True, size=B).astype(np.int64)
        else:
            lengths = np.full(B, int(L), dtype=np.int64)
        q_counts = np.ones(B, dtype=np.int64)
        q_pos = (lengths - 1).astype(np.int32)
        swa_pos0 = (lengths - W).astype(np.int32)
        swa_clip = None
    if "clip" in overrides and overrides["clip"] is not None:
        swa_clip = np.asarray(overrides["clip"], dtype=np.int32)
    T = int(q_counts.sum())
    N = int(lengths.sum())
    seq_start = np.zeros(B + 1, dtype=np.int64)
    seq_start[1:] = np.cumsum(lengths)
    q_start = np.zeros(B + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(q_counts)
    q_seq = np.repeat(np.arange(B), q_counts)

    cand = None
    if n_cand is not None:
        cand = np.empty((T, n_cand), dtype=np.int32)
        for b in range(B):
            n = int(lengths[b])
            m = min(n_cand, n)
            sel = np.sort(rng_len.choice(n, size=m, replace=False)).astype(np.int32)
            row = np.concatenate([sel, np.arange(m, n_cand, dtype=np.int64) + n]).astype(np.int32)
            cand[q_start[b]:q_start[b + 1]] = row
        max_ctx = n_cand
    else:
        max_ctx = int(q_pos.max()) + 1

    # peaked indexer keys: floor(frac * n) positions per sequence get +3 on every coordinate
    peak_rows = None
    if p["peak_frac"] > 0:
        rows = []
        for b in range(B):
            n = int(lengths[b])
            m = int(math.floor(p["peak_frac"] * n))
            rows.append(seq_start[b] + rng_peak.choice(n, size=m, replace=False))
        peak_rows = torch.as_tensor(np.sort(np.concatenate(rows)), device=device)

    dev = torch.device(device)
    # ---- indexer ----
    g = _torch_gen(ch[0], dev)
    qI = encode_e4m3(torch.randn((T, Hi, Di), generator=g, device=dev, dtype=torch.float32))
    g = _torch_gen(ch[1], dev)
    w = torch.rand((T, Hi), generator=g, device=dev, dtype=torch.float32)
    g = _torch_gen(ch[2], dev)
    kI = torch.empty((N, Di), dtype=torch.uint8, device=dev)

    def put_keys(r0, x):
        if peak_rows is not None:
            r1 = r0 + x.shape[0]
            lo = torch.searchsorted(peak_rows, torch.tensor(r0, device=dev))
            hi = torch.searchsorted(peak_rows, torch.tensor(r1, device=dev))
            sel = peak_rows[lo:hi] - r0
            x[sel] += 3.0
        kI[r0:r0 + x.shape[0]] = encode_e4m3(x)
    _randn_rows(g, N, Di, dev, put_keys)

    # ---- attention ----
    g = _torch_gen(ch[3], dev)
    q = torch.randn((T, Hq, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    g = _torch_gen(ch[4], dev)
    kv_codes = torch.empty((N, D // 2), dtype=torch.uint8, device=dev)
    kv_e8m0 = torch.empty((N, D // 32), dtype=torch.uint8, device=dev)
    kv_rowscale = torch.empty((N,), dtype=torch.float32, device=dev) if p["rowscale"] else None

    def put_latent(r0, x):
        c, e, rho = encode_mx_e2m1(x, p["rowscale"])
        r1 = r0 + x.shape[0]
        kv_codes[r0:r1] = c
        kv_e8m0[r0:r1] = e
        if rho is not None:
            kv_rowscale[r0:r1] = rho
    _randn_rows(g, N, D, dev, put_latent)

    g = _torch_gen(ch[5], dev)
    swa = torch.stack([encode_e4m3(torch.randn((W, D), generator=g, device=dev,
                                               dtype=torch.float32)) for _ in range(B)])

    t = lambda a, dt: torch.as_tensor(a, dtype=dt, device=dev)
    return Workload(
        name=name, B=B, T=T, Hi=Hi, Di=Di, k=k, Hq=Hq, D=D, W=W,
        sm_scale=1.0 / math.sqrt(D), max_ctx=max_ctx,
        seq_start=t(seq_start, torch.int64), q_start=t(q_start, torch.int32),
        q_pos=t(q_pos, torch.int32), qI=qI, w=w, kI=kI, kscale=None, q=q,
        kv_codes=kv_codes, kv_e8m0=kv_e8m0, kv_rowscale=kv_rowscale,
        swa=swa, swa_scale=None, swa_pos0=t(swa_pos0, torch.int32),
        swa_clip=None if swa_clip is None else t(swa_clip, torch.int32),
        cand=None if cand is None else t(cand, torch.int32),
        meta=dict(seed=seed, lengths=lengths.tolist(), q_seq=q_seq.tolist(), params=p),
    )


def encode_fp8_rows(x: torch.Tensor):
    """float32 rows [R, D] -> (E4M3 bytes [R, D], fp32 row scale [R]): each row is divided
    by rho = amax|row| / 448 (1 for a zero row) and rounded to E4M3."""
    amax = x.abs().amax(dim=1)
    rho = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    return encode_e4m3(x / rho[:, None]), rho


def with_fp8_kv(wl: Workload, seed: int = 2, rowscale: bool = True) -> Workload:
    """Attach an FP8 global latent cache of the same shape (fresh N(0,1) rows, E4M3 with a
    row scale, or without one the N(0,1) values rounded to E4M3 as they are): the input of
    the FP8-KV baseline attention."""
    dev = wl.kI.device
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    kv = torch.empty((wl.N, wl.D), dtype=torch.uint8, device=dev)
    rho = torch.empty((wl.N,), dtype=torch.float32, device=dev)

    def put(r0, x):
        c, r = encode_fp8_rows(x) if rowscale else (encode_e4m3(x), None)
        kv[r0:r0 + x.shape[0]] = c
        if rowscale:
            rho[r0:r0 + x.shape[0]] = r
    _randn_rows(g, wl.N, wl.D, dev, put)
    return dataclasses.replace(wl, kv_fp8=kv, kv_fp8_scale=rho if rowscale else None)


def encode_nvfp4(x: torch.Tensor, g: float):
    """float32 rows [R, D] -> (E2M1 codes uint8 [R, D/2], E4M3 scales uint8 [R, D/16]) for
    tensor scale g: each 16-element block gets the E4M3 scale s = RNE(amax / 6 / g) and its
    elements are rounded to E2M1 after division by s * g (0 for an all-zero block)."""
    R, D = x.shape
    assert D % 16 == 0
    blocks = x.view(R, D // 16, 16)
    bmax = blocks.abs().amax(dim=2)
    sc = encode_e4m3(bmax / 6.0 / g)
    sv = sc.view(torch.float8_e4m3fn).to(torch.float32) * g
    y = torch.where(sv[..., None] > 0, blocks / sv[..., None], torch.zeros_like(blocks))
    codes = _e2m1_round(y).view(R, D).to(torch.int32)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).to(torch.uint8)
    return packed, sc


def with_nvfp4_kv(wl: Workload, seed: int = 3, g: float = 2.0 ** -8) -> Workload:
    """Attach a global latent cache in the NVFP4 layout (fresh N(0,1) rows, tensor scale g)."""
    dev = wl.kI.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    codes = torch.empty((wl.N, wl.D // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((wl.N, wl.D // 16), dtype=torch.uint8, device=dev)

    def put(r0, x):
        c, sc = encode_nvfp4(x, g)
        codes[r0:r0 + x.shape[0]] = c
        scales[r0:r0 + x.shape[0]] = sc
    _randn_rows(gen, wl.N, wl.D, dev, put)
    return dataclasses.replace(wl, kv_nv_codes=codes, kv_nv_scales=scales, kv_nv_global=g)


def with_scales(wl: Workload, seed: int = 1) -> Workload:
    """Attach positive random per-key and per-window-row scales (exercise the optional inputs)."""
    g = torch.Generator(device=wl.kI.device)
    g.manual_seed(seed)
    dev = wl.kI.device
    kscale = 0.5 + torch.rand((wl.N,), generator=g, device=dev, dtype=torch.float32)
    swa_scale = 0.5 + torch.rand((wl.B, wl.W), generator=g, device=dev, dtype=torch.float32)
    return dataclasses.replace(wl, kscale=kscale, swa_scale=swa_scale)
