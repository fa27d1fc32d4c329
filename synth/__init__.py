"""Seeded synthetic inputs for the loss-scaling / FP8 workloads.

This module only produces input bit patterns.  It holds none of the method's
arithmetic (no unscale, no scale, no cast) and imports neither the oracle nor
the HIP library; tests and the benchmark feed its output to both.

Every generator is a pure function of (seed, stream, flat element index),
built from a counter-based 32-bit hash and integer operations only, plus
single IEEE-754 FP32 multiplications of exactly representable integers.
Because of that the same call gives the same bits on the CPU and on the GPU,
so a large tensor can be generated on the device while the oracle
regenerates any sampled subset of it on the host.

Hash: lowbias32 (Chris Wellons, "Prospecting for Hash Functions", 2018):
    x ^= x >> 16; x *= 0x7feb352d; x ^= x >> 15; x *= 0x846ca68b; x ^= x >> 16
applied twice over (index, key).  Products are formed from 16-bit halves
so no int64 intermediate overflows.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

M32 = 0xFFFFFFFF


# ------------------------------------------------------------------ hashing
def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & M32


def mix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _mix32_int(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def key(seed: int, stream: int, lane: int) -> int:
    return _mix32_int(_mix32_int(_mix32_int(seed) ^ (stream * 0x9E3779B9)) ^ (lane * 0x85EBCA6B))


def hash_u32(seed: int, stream: int, idx: torch.Tensor, lane: int = 0) -> torch.Tensor:
    """Uniform 32-bit words (int64 tensor in [0, 2^32)) for flat indices."""
    k = key(seed, stream, lane)
    lo = idx & M32
    hi = (idx >> 32) & M32
    return mix32(mix32(lo ^ k) ^ (hi * 0x27D4EB2F & M32) ^ ((k * 0x165667B1) & M32))


# ------------------------------------------------------------------ value recipes
def fp16_loguniform(seed: int, stream: int, idx: torch.Tensor, log2_lo: float,
                    log2_hi: float) -> torch.Tensor:
    """FP16 bit patterns (int64) with a fair sign and a log-uniform magnitude
    on [2^log2_lo, 2^log2_hi): a uniform "virtual log2" with 10 fraction bits
    is read as exponent.fraction (the piecewise-linear log of the binary
    format), and values below FP16's normal range become subnormals by
    shifting the significand right (truncating)."""
    u = hash_u32(seed, stream, idx, 1)
    s = hash_u32(seed, stream, idx, 2) >> 31
    lo_f = int(math.floor(log2_lo * 1024))
    span = int(math.floor(log2_hi * 1024)) - lo_f
    L = lo_f + ((u * span) >> 32)                      # fixed point, 10 fraction bits
    e = torch.div(L, 1024, rounding_mode="floor")
    m = L - e * 1024
    normal = ((e + 15) << 10) | m
    shift = (-14 - e).clamp(min=0, max=31)
    sub = (1024 + m) >> shift
    bits = torch.where(e >= -14, normal, sub)
    bits = torch.where(e >= 16, torch.full_like(bits, 0x7BFF), bits)
    return bits | (s << 15)


def _f32_to_bf16_rne(f: torch.Tensor) -> torch.Tensor:
    """BF16 bits of finite FP32 values, round to nearest even (integer ops)."""
    b = f.view(torch.int32).to(torch.int64) & M32
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF


def gaussian_f32(seed: int, stream: int, idx: torch.Tensor, sigma: float) -> torch.Tensor:
    """Approximately N(0, sigma^2) in FP32: the centred sum of four uniform
    16-bit integers (Irwin-Hall, bounded at +-3.46 sigma), times one FP32
    constant."""
    a = hash_u32(seed, stream, idx, 3)
    b = hash_u32(seed, stream, idx, 4)
    tot = (a & 0xFFFF) + (a >> 16) + (b & 0xFFFF) + (b >> 16)
    z = (2 * tot - 4 * 65535).to(torch.float32)          # exact: |z| < 2^19
    sd = math.sqrt(4 * (65536.0 ** 2 - 1) / 12.0) * 2.0   # std of 2*tot
    c = torch.tensor(sigma / sd, dtype=torch.float32, device=idx.device)
    return z * c


def laplace_f32(seed: int, stream: int, idx: torch.Tensor, b: float) -> torch.Tensor:
    """Laplace-shaped FP32 values with scale b: |x| = b ln2 (K + F) with K the
    number of trailing one bits of a uniform word (geometric, p = 1/2) and F
    uniform on [0, 1) with 18 bits; a fair sign."""
    u = hash_u32(seed, stream, idx, 5)
    v = hash_u32(seed, stream, idx, 6)
    K = torch.zeros_like(u)
    alive = torch.ones_like(u)
    for j in range(24):
        alive = alive & ((u >> j) & 1)
        K = K + alive
    mag = (K << 18) + (v & 0x3FFFF)                      # < 2^24: exact in FP32
    c = torch.tensor(b * math.log(2.0) / 2.0 ** 18, dtype=torch.float32, device=idx.device)
    x = mag.to(torch.float32) * c
    sign = (v >> 31).to(torch.bool)
    return torch.where(sign, -x, x)


def bernoulli(seed: int, stream: int, idx: torch.Tensor, p: float, lane: int = 7) -> torch.Tensor:
    thr = int(p * 2 ** 32)
    return hash_u32(seed, stream, idx, lane) < thr


def bf16_bits(f: torch.Tensor) -> torch.Tensor:
    return _f32_to_bf16_rne(f)


def to_bf16_tensor(bits: torch.Tensor) -> torch.Tensor:
    return bits.to(torch.int32).to(torch.int16).view(torch.bfloat16)


def to_f16_tensor(bits: torch.Tensor) -> torch.Tensor:
    return bits.to(torch.int32).to(torch.int16).view(torch.float16)


def as_u16_numpy(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ workloads
@dataclass
class GradSpec:
    """One FP16 gradient tensor of a multi-tensor gradient set."""
    name: str
    numel: int
    stream: int


@dataclass
class GradSet:
    seed: int
    scale: float                   # the loss scale S the stored values carry
    log2_lo: float                 # magnitude range of the stored FP16 values
    log2_hi: float
    tensors: list = field(default_factory=list)
    # step -> list of (tensor index, element index, FP16 bits) written before
    # that step and restored after it
    injections: dict = field(default_factory=dict)
    steps: int = 1

    def gen(self, t: int, idx: torch.Tensor) -> torch.Tensor:
        sp = self.tensors[t]
        return fp16_loguniform(self.seed, sp.stream, idx, self.log2_lo, self.log2_hi)

    def full(self, t: int, device) -> torch.Tensor:
        n = self.tensors[t].numel
        out = torch.empty(n, dtype=torch.float16, device=device)
        bits16 = out.view(torch.int16)
        step = 1 << 27
        for lo in range(0, n, step):
            idx = torch.arange(lo, min(n, lo + step), dtype=torch.int64, device=device)
            # an int64 -> int16 converting copy keeps the low 16 bits (an
            # elementwise kernel, not a device-to-device memcpy)
            bits16[lo:lo + idx.numel()].copy_(self.gen(t, idx))
        return out

    @property
    def total(self) -> int:
        return sum(s.numel for s in self.tensors)


INF16, NAN16 = 0x7C00, 0x7E00


def tiny_gradset() -> GradSet:
    """16 FP16 tensors of seeded sizes summing to 2^20 (most sizes not a
    multiple of 8); stored values carry S = 65536 and true magnitudes
    10^U(-9, -2); +Inf in tensor 5 before steps 3 and 7, NaN before step 20;
    50 steps."""
    rng = np.random.default_rng(1001)
    cuts = np.sort(rng.choice(np.arange(1, 1 << 20), size=15, replace=False))
    bounds = np.concatenate([[0], cuts, [1 << 20]])
    sizes = np.diff(bounds).tolist()
    S = 65536.0
    gs = GradSet(seed=1001, scale=S, log2_lo=math.log2(1e-9 * S), log2_hi=math.log2(1e-2 * S),
                 steps=50)
    gs.tensors = [GradSpec("g%d" % i, int(n), 100 + i) for i, n in enumerate(sizes)]
    pos = int(rng.integers(0, sizes[5]))
    gs.injections = {3: [(5, pos, INF16)], 7: [(5, pos, INF16)], 20: [(5, pos, NAN16)]}
    return gs


def llama3_8b_gradset() -> GradSet:
    """Llama-3-8B-shaped gradient set: embedding 128256x4096; 32 layers of
    q 4096x4096, k 1024x4096, v 1024x4096, o 4096x4096, gate/up 14336x4096,
    down 4096x14336 and two 4096 norms; final norm; untied lm_head
    128256x4096: 291 tensors, 8,030,261,248 elements.  True magnitudes
    log-uniform on [1e-10, 1e-1], stored x 2^15.  10 steps; +Inf at a seeded
    element of lm_head before step 2."""
    S = 2.0 ** 15
    gs = GradSet(seed=4004, scale=S, log2_lo=math.log2(1e-10 * S), log2_hi=math.log2(1e-1 * S),
                 steps=10)
    specs = [("embed", 128256 * 4096)]
    for l in range(32):
        specs += [("l%d.q" % l, 4096 * 4096), ("l%d.k" % l, 1024 * 4096),
                  ("l%d.v" % l, 1024 * 4096), ("l%d.o" % l, 4096 * 4096),
                  ("l%d.gate" % l, 14336 * 4096), ("l%d.up" % l, 14336 * 4096),
                  ("l%d.down" % l, 4096 * 14336), ("l%d.attn_norm" % l, 4096),
                  ("l%d.mlp_norm" % l, 4096)]
    specs += [("norm", 4096), ("lm_head", 128256 * 4096)]
    gs.tensors = [GradSpec(n, k, 4000 + i) for i, (n, k) in enumerate(specs)]
    rng = np.random.default_rng(4004)
    gs.injections = {2: [(len(specs) - 1, int(rng.integers(0, 128256 * 4096)), INF16)]}
    return gs


@dataclass
class QuantSpec:
    """One 2-D BF16 tensor to quantize."""
    name: str
    rows: int
    cols: int
    fmt: int                       # 0 = E4M3, 1 = E5M2
    gran: int                      # 0 per-tensor, 1 = 1x128, 2 = 128x128
    seed: int
    stream: int
    kind: str                      # "gauss" | "laplace"
    sigma: float
    outlier_p: float = 0.0
    outlier_mult: float = 1.0

    def gen_f32(self, idx: torch.Tensor) -> torch.Tensor:
        if self.kind == "gauss":
            f = gaussian_f32(self.seed, self.stream, idx, self.sigma)
        else:
            f = laplace_f32(self.seed, self.stream, idx, self.sigma)
        if self.outlier_p > 0:
            m = bernoulli(self.seed, self.stream, idx, self.outlier_p)
            mult = torch.tensor(self.outlier_mult, dtype=torch.float32, device=idx.device)
            f = torch.where(m, f * mult, f)
        return f

    def gen(self, idx: torch.Tensor) -> torch.Tensor:
        """BF16 bit patterns (int64) of the flat elements idx."""
        return bf16_bits(self.gen_f32(idx))

    def full(self, device) -> torch.Tensor:
        n = self.rows * self.cols
        out = torch.empty(n, dtype=torch.bfloat16, device=device)
        bits16 = out.view(torch.int16)
        step = 1 << 27
        for lo in range(0, n, step):
            idx = torch.arange(lo, min(n, lo + step), dtype=torch.int64, device=device)
            bits16[lo:lo + idx.numel()].copy_(self.gen(idx))
        return out.view(self.rows, self.cols)


def tiny_quant() -> QuantSpec:
    """1024x1024 BF16 N(0,1), per-tensor E4M3."""
    return QuantSpec("act1024", 1024, 1024, 0, 0, 1001, 200, "gauss", 1.0)


def per_tensor_at_scale() -> list:
    """8192x8192 BF16 N(0,1) with 0.1% of entries x1000 -> per-tensor E4M3;
    8192x8192 BF16 Laplace(0, 1e-4) -> per-tensor E5M2."""
    return [QuantSpec("act8192", 8192, 8192, 0, 0, 2002, 300, "gauss", 1.0, 0.001, 1000.0),
            QuantSpec("grad8192", 8192, 8192, 1, 0, 2002, 301, "laplace", 1e-4)]


def deepseek_v3_blocks() -> list:
    """Activations 16384x7168 BF16 N(0,1) -> 1x128 E4M3 (16384x56 scales);
    weights 7168x18432 BF16 N(0, 0.02) -> 128x128 E4M3 (56x144 scales);
    0.01% of entries x500 in both."""
    return [QuantSpec("act_1x128", 16384, 7168, 0, 1, 3003, 400, "gauss", 1.0, 1e-4, 500.0),
            QuantSpec("wgt_128x128", 7168, 18432, 0, 2, 3003, 401, "gauss", 0.02, 1e-4, 500.0)]


# ------------------------------------------------------------------ special values
def _bf16_from_f32_bits(b32: torch.Tensor) -> torch.Tensor:
    return ((b32 + 0x7FFF + ((b32 >> 16) & 1)) >> 16) & 0xFFFF


def special_mix_bits(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """BF16 bit patterns, class chosen per element by a hash:
    90% N(0,1) (Irwin-Hall); 2% NaN (random sign and payload); 2% +-Inf;
    2% magnitudes 2^U(-24,-14) (FP16-subnormal range); 2% +-0; 1% just above
    the FP8 maxima (BF16 values 450..480 and 57600..61440); 1% exact
    E4M3/E5M2 midpoints at scale 1 (a BF16 whose fraction is an FP8 fraction
    plus one half unit)."""
    cls = hash_u32(seed, stream, idx, 11) % 100
    u = hash_u32(seed, stream, idx, 12)
    sign = (u >> 31) << 15
    g = bf16_bits(gaussian_f32(seed, stream, idx, 1.0))
    nan = sign | 0x7F80 | (1 + (u % 127))
    inf = sign | 0x7F80
    # log-uniform over [2^-24, 2^-14): BF16 exponent field 103..112
    tiny = sign | ((103 + (u >> 8) % 10) << 7) | (u & 0x7F)
    zero = sign
    # just above 448 (0x43E0) or 57344 (0x4760): BF16 neighbours 1..16 ulps up
    above = sign | torch.where(((u >> 9) & 1) == 1, 0x43E0 + 1 + (u & 0xF), 0x4760 + 1 + (u & 0xF))
    # midpoints: E4M3 (fraction bit 3 set below 3 FP8 fraction bits) in the
    # E4M3 normal range, or E5M2 (bit 4 below 2 fraction bits) in its range
    e4 = ((121 + (u >> 4) % 15) << 7) | (((u >> 1) & 7) << 4) | 0x8
    e5 = ((113 + (u >> 4) % 30) << 7) | (((u >> 1) & 3) << 5) | 0x10
    mid = sign | torch.where((u & 1) == 1, e4, e5)
    out = g
    out = torch.where(cls >= 90, nan, out)
    out = torch.where(cls >= 92, inf, out)
    out = torch.where(cls >= 94, tiny, out)
    out = torch.where(cls >= 96, zero, out)
    out = torch.where(cls >= 98, above, out)
    out = torch.where(cls >= 99, mid, out)
    return out


def anchored_bits(seed: int, stream: int, idx: torch.Tensor, anchor: float = 448.0) -> torch.Tensor:
    """BF16 bit patterns where every 1x128 block holds one +-anchor*2^k
    (k seeded in [-8, 8]) as its largest magnitude, so a block scale derived
    from the amax is a power of two; the body is N(0, (anchor 2^k / 8)^2)
    clipped below the anchor, with 1/16 of the elements replaced by exact
    E4M3 / E5M2 midpoints relative to that power-of-two scale."""
    blk = idx >> 7
    pos = idx & 127
    hb = hash_u32(seed, stream, blk, 21)
    k = (hb % 17) - 8
    anchor_pos = (hb >> 8) & 127
    lg2a = int(math.log2(anchor))                   # 448 = 1.75 * 2^8; 57344 = 1.75 * 2^15
    a_exp = 127 + lg2a + k                           # FP32 exponent of anchor * 2^k
    anchor_f32 = (a_exp << 23) | 0x600000            # 1.75 * 2^(lg2a + k)
    body = gaussian_f32(seed, stream, idx, 1.0)
    # body scale 1.75 * 2^(lg2a + k - 3) = (anchor 2^k) / 8, built from its bits
    scale = (((a_exp - 3) << 23) | 0x600000).to(torch.int32).view(torch.float32)
    b = body * scale
    lim = anchor_f32.to(torch.int32).view(torch.float32) * torch.tensor(0.99, device=idx.device)
    b = torch.maximum(torch.minimum(b, lim), -lim)
    bits = bf16_bits(b)
    u = hash_u32(seed, stream, idx, 22)
    # s = anchor*2^k / MAX = 2^k (E4M3, anchor 448): midpoint m * 2^k
    e_m = (127 + k - 3 + (u >> 4) % 10)
    mid = ((u >> 31) << 15) | (e_m << 7) | (((u >> 1) & 7) << 4) | 0x8
    bits = torch.where((u % 16) == 0, mid, bits)
    a_bits = ((hb >> 31) << 15) | (anchor_f32 >> 16)
    return torch.where(pos == anchor_pos, a_bits, bits)


def saturation_bits(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """BF16 values uniform in [0.9, 1.2] x MAX of E4M3 or E5M2 (chosen per
    element), random sign, and 1% +-Inf."""
    u = hash_u32(seed, stream, idx, 31)
    v = hash_u32(seed, stream, idx, 32)
    frac = (v & 0xFFFFFF).to(torch.float32) * torch.tensor(2.0 ** -24 * 0.3, device=idx.device)
    m = torch.where((u & 1) == 1, torch.tensor(448.0, device=idx.device),
                    torch.tensor(57344.0, device=idx.device))
    f = (frac + 0.9) * m
    bits = bf16_bits(f) | ((u >> 31) << 15)
    inf = ((u >> 30) & 1) << 15 | 0x7F80
    return torch.where((u >> 8) % 100 == 0, inf, bits)


def random_bits(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """Uniformly random 16-bit patterns (NaN, Inf and subnormals included)."""
    return hash_u32(seed, stream, idx, 41) & 0xFFFF


@dataclass
class BitsSpec:
    """A 2-D BF16 tensor given by a bit-pattern generator."""
    name: str
    rows: int
    cols: int
    seed: int
    stream: int
    kind: str                      # "mix" | "anchored" | "saturation" | "random"

    def gen(self, idx: torch.Tensor) -> torch.Tensor:
        if self.kind == "mix":
            return special_mix_bits(self.seed, self.stream, idx)
        if self.kind == "anchored":
            return anchored_bits(self.seed, self.stream, idx)
        if self.kind == "saturation":
            return saturation_bits(self.seed, self.stream, idx)
        return random_bits(self.seed, self.stream, idx)

    def full(self, device) -> torch.Tensor:
        n = self.rows * self.cols
        out = torch.empty(n, dtype=torch.bfloat16, device=device)
        bits16 = out.view(torch.int16)
        step = 1 << 27
        for lo in range(0, n, step):
            idx = torch.arange(lo, min(n, lo + step), dtype=torch.int64, device=device)
            bits16[lo:lo + idx.numel()].copy_(self.gen(idx))
        return out.view(self.rows, self.cols)


def special_values_4gib() -> list:
    """Four 16384x32768 BF16 tensors (2^31 elements, 4 GiB): class mix,
    anchored blocks, saturation edge, random bit patterns."""
    return [BitsSpec("mix", 16384, 32768, 5005, 500, "mix"),
            BitsSpec("anchored", 16384, 32768, 5005, 501, "anchored"),
            BitsSpec("saturation", 16384, 32768, 5005, 502, "saturation"),
            BitsSpec("random", 16384, 32768, 5005, 503, "random")]
