"""Seeded synthetic inputs for the routed MoE layer.

This module draws inputs only; it holds none of the layer's arithmetic (no
format decoding, no routing, no GEMM).  Both the GPU path and the CPU oracle
take their inputs from here, so that the two see the same bytes.

Random source: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), evaluated as a counter-based generator:
output i of stream ``key`` is ``mix64(key + (i + 1) * GOLDEN)`` with the
published finaliser ``mix64``.  Every element is addressable by index, so a
single expert, a single token or a whole tensor can be drawn on any device
and the bytes are identical.

Distributions (one per tensor):
  x          bf16 ~ N(0, 1)        Box-Muller on two 32-bit halves, fp64,
                                    rounded to fp32 then to bf16;
  router_w   bf16 ~ N(0, 0.02^2)   same recipe, scaled by 0.02;
  codes      uniform bytes, i.e. both E2M1 nibbles uniform over 16 codes;
  scales     E8M0 codes uniform over 123..127 (scales 2^-4 .. 2^0);
  bias       Zipf-style skew b_e = -beta * s * ln(e + 1) (s = 1.1) for the
             skewed prefill workload, none elsewhere;
  FP8 experts: E4M3FN codes uniform bytes with the two NaN codes (0x7F,
             0xFF) moved to their neighbours +-448 (0x7E, 0xFE); one fp32
             scale per 128 x 128 block, (1 + u) * 2^-8 with u uniform on a
             24-bit grid in [0, 1);
  MoE tail (pre-norm block): gamma bf16 = 1 + N(0, 0.1^2) (RMSNorm weight),
             eps = 1e-6, one shared expert of width f with bf16 gate/up
             [2f][d] and down [d][f] weights ~ N(0, 1).

Integer draws are exact on every device.  The normal draws use fp64
log/sqrt/cos, which may differ in the last ulp between CPU builds; they are
therefore always drawn on the CPU and copied to the device.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

TENSOR_X, TENSOR_WR, TENSOR_GU_CODES, TENSOR_GU_SCALES = 1, 2, 3, 4
TENSOR_DN_CODES, TENSOR_DN_SCALES = 5, 6
TENSOR_GAMMA, TENSOR_SHARED_GU, TENSOR_SHARED_DN = 7, 8, 9
TENSOR_FP8_GU_CODES, TENSOR_FP8_GU_SCALES, TENSOR_FP8_DN_CODES, TENSOR_FP8_DN_SCALES = 10, 11, 12, 13
TAIL_EPS = 1e-6

SCALE_CODE_LO, SCALE_CODE_N = 123, 5      # E8M0 codes 123..127


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    T: int
    d: int
    E: int
    k: int
    f: int
    seed: int
    batches: int = 1          # distinct seeded batches (decode: tokens)
    zipf_beta: float = 0.0    # 0 -> no router bias
    zipf_s: float = 1.1
    wfmt: str = "mxfp4"       # expert store: "mxfp4" or "fp8" (E4M3FN + 128x128 fp32 scales)
    notes: str = field(default="", compare=False)

    @property
    def rows(self) -> int:
        return self.T * self.k

    @property
    def expert_bytes(self) -> int:
        d, f = self.d, self.f
        if self.wfmt == "fp8":
            return 3 * d * f + 4 * (2 * f // 128) * (d // 128) + 4 * (d // 128) * (f // 128)
        return 2 * f * (d // 2) + 2 * f * (d // 32) + d * (f // 2) + d * (f // 32)

    @property
    def gate_up_bytes(self) -> int:
        d, f = self.d, self.f
        if self.wfmt == "fp8":
            return 2 * f * d + 4 * (2 * f // 128) * (d // 128)
        return 2 * f * (d // 2) + 2 * f * (d // 32)


# The workloads: tiny parity layer, one-token decode (1000 tokens), 64-token
# batched decode, 4096-token skewed prefill, 32768-token prefill; and the
# same layer at a second routing shape, one-token decode and prefill.
CONFIGS = {
    0: Config(0, "tiny T=8 d=256 E=16 k=2 f=128", 8, 256, 16, 2, 128, seed=0),
    1: Config(1, "decode T=1 d=7168 E=896 k=16 f=1536 x1000 tokens", 1, 7168,
              896, 16, 1536, seed=1, batches=1000),
    2: Config(2, "batched decode T=64 d=7168 E=896 k=16 f=1536", 64, 7168, 896,
              16, 1536, seed=2, batches=50),
    # beta bisected so that the hottest expert gets 9.5-10.5x the mean load
    # under the canonical routing (9.98x: 730 rows against 73.1; the
    # coldest gets 20) -- tests/golden/zipf_beta.py, zipf_beta.json
    3: Config(3, "zipf prefill T=4096 d=7168 E=896 k=16 f=1536", 4096, 7168,
              896, 16, 1536, seed=3, zipf_beta=0.3375),
    4: Config(4, "long prefill T=32768 d=7168 E=896 k=16 f=1536", 32768, 7168,
              896, 16, 1536, seed=4),
    # a second routing shape: 256 experts, top-8 (MiMo V2.6 Flash); d and f
    # are synthetic (d * f ~ 310e9 / (48 layers * 256 experts * 3))
    5: Config(5, "mimo decode T=1 d=4096 E=256 k=8 f=2048 x1000 tokens", 1, 4096,
              256, 8, 2048, seed=5, batches=1000),
    6: Config(6, "mimo prefill T=4096 d=4096 E=256 k=8 f=2048", 4096, 4096, 256, 8,
              2048, seed=6),
    # the K3 shape with FP8 experts (E4M3FN, fp32 scale per 128 x 128 block)
    7: Config(7, "fp8 decode T=1 d=7168 E=896 k=16 f=1536 x1000 tokens", 1, 7168, 896, 16,
              1536, seed=7, batches=1000, wfmt="fp8"),
    8: Config(8, "fp8 zipf prefill T=4096 d=7168 E=896 k=16 f=1536", 4096, 7168, 896, 16,
              1536, seed=8, zipf_beta=0.34, wfmt="fp8"),
}


# ---------------------------------------------------------------------------
# SplitMix64
# ---------------------------------------------------------------------------
def mix64_int(z: int) -> int:
    """Published SplitMix64 finaliser on a Python int (mod 2^64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def splitmix64_int(key: int, i: int) -> int:
    """Output i of the stream seeded with ``key`` (pure-Python reference)."""
    return mix64_int((key + (i + 1) * GOLDEN) & MASK64)


def stream_key(seed: int, tensor: int, batch: int = 0) -> int:
    """Key of one tensor's stream: a hash of (seed, tensor id, batch)."""
    k = mix64_int(seed * 0x100000001B3 + 0x5EED)
    k = mix64_int(k ^ (tensor * 0xD6E8FEB86659FD93))
    return mix64_int(k ^ (batch * 0xA0761D6478BD642F + 1))


def _s64(u: int) -> int:
    u &= MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)


def splitmix64(counters: torch.Tensor, key: int) -> torch.Tensor:
    """Outputs (as int64 bit patterns) at the given int64 counters."""
    z = counters * _s64(GOLDEN) + _s64(key + GOLDEN)
    z = (z ^ _lsr(z, 30)) * _s64(MIX1)
    z = (z ^ _lsr(z, 27)) * _s64(MIX2)
    return z ^ _lsr(z, 31)


# ---------------------------------------------------------------------------
# Draws
# ---------------------------------------------------------------------------
def _arange(start: int, n: int, device) -> torch.Tensor:
    return torch.arange(start, start + n, dtype=torch.int64, device=device)


def random_bytes(key: int, start_byte: int, n_bytes: int, device="cpu"):
    """Bytes [start_byte, start_byte + n_bytes) of a stream; both bounds must
    be multiples of 8 (each 64-bit output gives 8 little-endian bytes)."""
    assert start_byte % 8 == 0 and n_bytes % 8 == 0
    z = splitmix64(_arange(start_byte // 8, n_bytes // 8, device), key)
    return z.view(torch.uint8)


def scale_codes(key: int, start: int, n: int, device="cpu"):
    """E8M0 codes uniform over 123..127, one stream output per code."""
    z = splitmix64(_arange(start, n, device), key)
    pick = (_lsr(z, 32) * SCALE_CODE_N) >> 32          # 0..4
    return (pick + SCALE_CODE_LO).to(torch.uint8)


def normals_bf16(key: int, start: int, n: int, sigma: float,
                 chunk: int = 1 << 24) -> torch.Tensor:
    """n bf16 draws of N(0, sigma^2) on the CPU (Box-Muller, fp64)."""
    out = torch.empty(n, dtype=torch.bfloat16)
    for c0 in range(0, n, chunk):
        m = min(chunk, n - c0)
        z = splitmix64(_arange(start + c0, m, "cpu"), key)
        hi = _lsr(z, 32).to(torch.float64)
        lo = (z & 0xFFFFFFFF).to(torch.float64)
        u1 = (hi + 1.0) * (1.0 / 4294967296.0)          # (0, 1]
        u2 = lo * (1.0 / 4294967296.0)                  # [0, 1)
        g = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
        out[c0:c0 + m] = (g * sigma).to(torch.float32).to(torch.bfloat16)
    return out


def gen_x(cfg: Config, batch: int = 0, tokens=None) -> torch.Tensor:
    """Activations [T][d] bf16 on the CPU for one batch; ``tokens`` (a range
    or list) draws only those rows."""
    key = stream_key(cfg.seed, TENSOR_X, batch)
    if tokens is None:
        return normals_bf16(key, 0, cfg.T * cfg.d, 1.0).view(cfg.T, cfg.d)
    rows = [normals_bf16(key, t * cfg.d, cfg.d, 1.0) for t in tokens]
    return torch.stack(rows) if rows else torch.empty(0, cfg.d, dtype=torch.bfloat16)


def gen_router_w(cfg: Config) -> torch.Tensor:
    key = stream_key(cfg.seed, TENSOR_WR)
    return normals_bf16(key, 0, cfg.E * cfg.d, 0.02).view(cfg.E, cfg.d)


def gen_bias(cfg: Config):
    """Router bias [E] fp32, or None when the workload has no skew."""
    if cfg.zipf_beta == 0.0:
        return None
    e = torch.arange(cfg.E, dtype=torch.float64)
    return (-cfg.zipf_beta * cfg.zipf_s * torch.log(e + 1.0)).to(torch.float32)


def expert_sizes(cfg: Config) -> dict:
    d, f = cfg.d, cfg.f
    return {"gu_codes": (2 * f, d // 2), "gu_scales": (2 * f, d // 32),
            "dn_codes": (d, f // 2), "dn_scales": (d, f // 32)}


def gen_experts(cfg: Config, experts=None, device="cpu",
                chunk_experts: int = 32) -> dict:
    """MXFP4 expert tensors for the listed experts (default: all), stacked in
    the listed order: gu_codes [n][2f][d/2], gu_scales [n][2f][d/32],
    dn_codes [n][d][f/2], dn_scales [n][d][f/32] (uint8)."""
    if experts is None:
        experts = range(cfg.E)
    experts = list(experts)
    n = len(experts)
    sizes = expert_sizes(cfg)
    out = {name: torch.empty((n,) + shp, dtype=torch.uint8, device=device)
           for name, shp in sizes.items()}
    keys = {"gu_codes": stream_key(cfg.seed, TENSOR_GU_CODES),
            "gu_scales": stream_key(cfg.seed, TENSOR_GU_SCALES),
            "dn_codes": stream_key(cfg.seed, TENSOR_DN_CODES),
            "dn_scales": stream_key(cfg.seed, TENSOR_DN_SCALES)}
    for name, shp in sizes.items():
        per = shp[0] * shp[1]
        flat = out[name].view(n, per)
        # contiguous runs of expert ids are drawn in one go
        i = 0
        while i < n:
            j = i
            while (j + 1 < n and experts[j + 1] == experts[j] + 1
                   and j + 1 - i < chunk_experts):
                j += 1
            e0, cnt = experts[i], j - i + 1
            if name.endswith("codes"):
                v = random_bytes(keys[name], e0 * per, cnt * per, device)
            else:
                v = scale_codes(keys[name], e0 * per, cnt * per, device)
            flat[i:i + cnt] = v.view(cnt, per)
            i = j + 1
    return out


def fp8_expert_sizes(cfg: Config) -> dict:
    d, f = cfg.d, cfg.f
    return {"gu_codes": (2 * f, d), "gu_scales": (2 * f // 128, d // 128),
            "dn_codes": (d, f), "dn_scales": (d // 128, f // 128)}


def gen_experts_fp8(cfg: Config, experts=None, device="cpu", chunk_experts: int = 32) -> dict:
    """FP8 expert tensors for the listed experts (default: all): gu_codes
    uint8 [n][2f][d], gu_scales fp32 [n][2f/128][d/128], dn_codes uint8
    [n][d][f], dn_scales fp32 [n][d/128][f/128].  Needs d, f % 128 == 0.
    Contiguous runs of expert ids are drawn in one go."""
    assert cfg.d % 128 == 0 and cfg.f % 128 == 0
    if experts is None:
        experts = range(cfg.E)
    experts = list(experts)
    n = len(experts)
    sizes = fp8_expert_sizes(cfg)
    keys = {"gu_codes": stream_key(cfg.seed, TENSOR_FP8_GU_CODES),
            "gu_scales": stream_key(cfg.seed, TENSOR_FP8_GU_SCALES),
            "dn_codes": stream_key(cfg.seed, TENSOR_FP8_DN_CODES),
            "dn_scales": stream_key(cfg.seed, TENSOR_FP8_DN_SCALES)}
    out = {}
    for name, shp in sizes.items():
        per = shp[0] * shp[1]
        codes = name.endswith("codes")
        t = torch.empty((n,) + shp, dtype=torch.uint8 if codes else torch.float32, device=device)
        flat = t.view(n, per)
        i = 0
        while i < n:
            j = i
            while (j + 1 < n and experts[j + 1] == experts[j] + 1
                   and j + 1 - i < chunk_experts):
                j += 1
            e0, cnt = experts[i], j - i + 1
            if codes:
                b = random_bytes(keys[name], e0 * per, cnt * per, device)
                flat[i:i + cnt] = torch.where((b & 0x7F) == 0x7F, b - 1, b).view(cnt, per)
            else:
                z = splitmix64(_arange(e0 * per, cnt * per, device), keys[name])
                u = _lsr(z, 40).to(torch.float64) * (1.0 / 16777216.0)     # 24-bit grid
                flat[i:i + cnt] = ((1.0 + u) * 2.0 ** -8).to(torch.float32).view(cnt, per)
            i = j + 1
        out[name] = t
    return out


def gen_layer(cfg: Config, batch: int = 0, device="cpu") -> dict:
    """Everything one layer call needs (x and router on the CPU are copied to
    ``device``)."""
    d = {"x": gen_x(cfg, batch).to(device),
         "router_w": gen_router_w(cfg).to(device),
         "bias": None}
    b = gen_bias(cfg)
    if b is not None:
        d["bias"] = b.to(device)
    d.update(gen_experts(cfg, device=device))
    return d


def gen_tail(cfg: Config, fs: int = 0, device="cpu") -> dict:
    """The MoE tail's weights: RMSNorm weight gamma [d] and one shared expert of
    width fs (default f): gate/up [2fs][d] and down [d][fs], all bf16, drawn on
    the CPU and copied to ``device``; eps is the norm's epsilon."""
    fs = fs or cfg.f
    d = cfg.d
    g = normals_bf16(stream_key(cfg.seed, TENSOR_GAMMA), 0, d, 0.1)
    gamma = (1.0 + g.to(torch.float32)).to(torch.bfloat16)
    sgu = normals_bf16(stream_key(cfg.seed, TENSOR_SHARED_GU), 0, 2 * fs * d, 1.0)
    sdn = normals_bf16(stream_key(cfg.seed, TENSOR_SHARED_DN), 0, d * fs, 1.0)
    return {"gamma": gamma.to(device), "eps": TAIL_EPS,
            "shared_gu": sgu.view(2 * fs, d).to(device),
            "shared_dn": sdn.view(d, fs).to(device)}


def as_u16(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit pattern (CPU copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")


def as_u8(t: torch.Tensor):
    return t.detach().to("cpu").contiguous().numpy()
