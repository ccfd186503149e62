"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and stores them in the operand formats; it
holds none of the product's arithmetic, so both the fp64 oracle and the HIP
path can read the very same bytes.  Every draw uses a CPU ``torch.Generator``
seeded explicitly, in the order A, B, then the scale tensors.

Workloads (sizes, formats and value distributions of the five measured
problems):

* ``tile_f16``   -- one tile, A 128x64 and B 64x64 float16, uniform [-1, 1],
  seed 0, float32 output (the single-CTA example of "Blackwell Tensor Cores",
  The Accumulator's Lifetime).
* ``bf16_4096``  -- A, B 4096x4096 bfloat16, N(0,1)*0.1, seed 1, bf16 output.
* ``batched``    -- 1024 problems of A 128x64, B 256x64 bfloat16, uniform
  [-1, 1], seed 2, float32 output (the 128x256x64 bf16 tile of "API Card:
  Blackwell Pipeline (tcgen05)", Descriptor.).
* ``bf16_8192``  -- A, B 8192x8192 bfloat16, N(0,1)*0.05, seed 3, bf16 output.
* ``mxfp8_8192`` -- A, B 8192x8192 E4M3 drawn N(0,1) then cast, one E8M0 scale
  per 32 K elements per row with exponents uniform on the integers -4..4,
  seed 4, bf16 output ("Hopper and Blackwell GEMM", block-scaling table).
* ``mxfp4_8192`` -- the same with E2M1 elements (MXFP4, the table's 4-bit
  row): every 4-bit code equally likely, seed 5, bf16 output.
* ``mxfp6_8192`` -- the same with FP6 E2M3 elements (MXFP6, the table's 6-bit
  rows): every 6-bit code equally likely, packed four per three bytes, seed
  7, bf16 output.
* ``nvfp4_8192`` -- A, B 8192x8192 E2M1 codes (every code equally likely),
  one E4M3 scale per 16 (exponent uniform on -4..4, every mantissa), tensor
  scales 0.5 and 1.25, seed 8, bf16 output (the format table's NVFP4 row).
* ``mxfp8_8192_mn`` -- MXFP8 8192^3 with A column-major (stored K x M, its M
  index contiguous) and B row-major (stored K x N): E4M3 N(0,1) elements and
  E8M0 scales as ``mxfp8_8192``, seed 9, bf16 output ("API Card: Blackwell
  Pipeline (tcgen05)", Descriptor.: fp8 types in either majorness).
* ``bf16_8192_nn`` -- A 8192x8192 and B 8192x8192 bfloat16, both row-major
  (B stored K x N, its N index contiguous: the product A . B of two
  row-major matrices), N(0,1)*0.05, seed 6, bf16 output ("API Card:
  Blackwell Pipeline (tcgen05)", Descriptor.: 16-bit types in either
  majorness).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

E8M0_BIAS = 127


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    M: int
    N: int
    K: int
    dtype: str          # "f16", "bf16", or "e4m3" / "e2m1" / "e2m3" / "e3m2" (MX block-scaled)
    out_dtype: str      # "f32" or "bf16"
    seed: int
    dist: str           # "uniform", "normal" or "codes" (every code equally likely)
    sigma: float = 1.0
    scale_exp: tuple = field(default=(-4, 4))
    b_order: str = "col"  # "col": B stored N x K (the TN form); "row": stored K x N
    a_order: str = "row"  # "row": A stored M x K (the TN form); "col": stored K x M
    globals: tuple = field(default=(1.0, 1.0))  # NVFP4 per-tensor scales gA, gB

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K


WORKLOADS = {
    "tile_f16": Workload("tile_f16", 1, 128, 64, 64, "f16", "f32", 0, "uniform"),
    "bf16_4096": Workload("bf16_4096", 1, 4096, 4096, 4096, "bf16", "bf16", 1, "normal", 0.1),
    "batched": Workload("batched", 1024, 128, 256, 64, "bf16", "f32", 2, "uniform"),
    "bf16_8192": Workload("bf16_8192", 1, 8192, 8192, 8192, "bf16", "bf16", 3, "normal", 0.05),
    "mxfp8_8192": Workload("mxfp8_8192", 1, 8192, 8192, 8192, "e4m3", "bf16", 4, "normal", 1.0),
    "mxfp4_8192": Workload("mxfp4_8192", 1, 8192, 8192, 8192, "e2m1", "bf16", 5, "codes"),
    "mxfp6_8192": Workload("mxfp6_8192", 1, 8192, 8192, 8192, "e2m3", "bf16", 7, "codes"),
    "nvfp4_8192": Workload("nvfp4_8192", 1, 8192, 8192, 8192, "nvfp4", "bf16", 8, "codes",
                           globals=(0.5, 1.25)),
    "bf16_8192_nn": Workload("bf16_8192_nn", 1, 8192, 8192, 8192, "bf16", "bf16", 6, "normal", 0.05,
                             b_order="row"),
    "mxfp8_8192_mn": Workload("mxfp8_8192_mn", 1, 8192, 8192, 8192, "e4m3", "bf16", 9, "normal", 1.0,
                              b_order="row", a_order="col"),
}

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def uniform(shape, gen, dtype) -> torch.Tensor:
    """Uniform on [-1, 1] drawn in float32, then rounded to ``dtype``."""
    return (torch.rand(shape, generator=gen, dtype=torch.float32) * 2 - 1).to(dtype)


def normal(shape, gen, sigma, dtype) -> torch.Tensor:
    """N(0, sigma^2) drawn in float32, then rounded to ``dtype``."""
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * sigma).to(dtype)


def e4m3_normal(shape, gen, sigma=1.0) -> torch.Tensor:
    """N(0, sigma^2) in float32, clamped to the E4M3 range, cast to E4M3; the
    bytes are returned as uint8."""
    x = torch.randn(shape, generator=gen, dtype=torch.float32) * sigma
    return x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def e2m1_codes(rows: int, k: int, gen) -> torch.Tensor:
    """rows x k E2M1 elements, every 4-bit code equally likely, stored two per
    byte (element 2t in the low four bits of byte t): uint8 of shape
    rows x k/2."""
    c = torch.randint(0, 16, (rows, k), generator=gen, dtype=torch.int32)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).to(torch.uint8)


def pack_fp6(codes: torch.Tensor) -> torch.Tensor:
    """6-bit codes (rows x k, k a multiple of 4) packed as one little-endian
    bit stream per row, element t in bits 6t .. 6t+5: uint8 rows x 3k/4."""
    c = codes.to(torch.int32)
    w = c[:, 0::4] | (c[:, 1::4] << 6) | (c[:, 2::4] << 12) | (c[:, 3::4] << 18)
    return torch.stack([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], dim=2).reshape(
        c.shape[0], -1).to(torch.uint8)


def fp6_codes(rows: int, k: int, gen) -> torch.Tensor:
    """rows x k FP6 elements (E2M3 or E3M2), every 6-bit code equally likely,
    packed by pack_fp6: uint8 of shape rows x 3k/4."""
    return pack_fp6(torch.randint(0, 64, (rows, k), generator=gen, dtype=torch.int32))


def e4m3_scales(shape, gen, lo=-4, hi=4) -> torch.Tensor:
    """Positive E4M3 scale bytes with exponent uniform on the integers lo..hi
    and every mantissa equally likely (NVFP4 block scales)."""
    e = torch.randint(lo, hi + 1, shape, generator=gen, dtype=torch.int32) + 7
    m = torch.randint(0, 8, shape, generator=gen, dtype=torch.int32)
    return ((e << 3) | m).to(torch.uint8)


def e8m0_scales(shape, gen, lo=-4, hi=4) -> torch.Tensor:
    """E8M0 bytes 127+s with s uniform on the integers lo..hi."""
    return (torch.randint(lo, hi + 1, shape, generator=gen, dtype=torch.int32)
            + E8M0_BIAS).to(torch.uint8)


def quarter_integers(shape, gen, dtype) -> torch.Tensor:
    """Values in {-1, -3/4, ..., 3/4, 1}: integers -4..4 divided by 4 (the input
    structure of the 16x8x32 example in "mma.sync", Examples)."""
    return (torch.randint(-4, 5, shape, generator=gen, dtype=torch.int32).float() / 4).to(dtype)


def make(w: Workload | str) -> dict:
    """CPU tensors for a workload: A, B (and SA, SB for MX)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    g = generator(w.seed)
    lead = (w.batch,) if w.batch > 1 else ()
    shp_a = lead + ((w.K, w.M) if w.a_order == "col" else (w.M, w.K))
    shp_b = lead + ((w.K, w.N) if w.b_order == "row" else (w.N, w.K))
    if w.dtype == "nvfp4":
        a, b = e2m1_codes(w.M, w.K, g), e2m1_codes(w.N, w.K, g)
        lo, hi = w.scale_exp
        return {"A": a, "B": b, "SA": e4m3_scales((w.M, w.K // 16), g, lo, hi),
                "SB": e4m3_scales((w.N, w.K // 16), g, lo, hi)}
    if w.dtype in ("e4m3", "e2m1", "e2m3", "e3m2"):
        if w.dtype == "e4m3":
            a = e4m3_normal(shp_a, g, w.sigma)
            b = e4m3_normal(shp_b, g, w.sigma)
        elif w.dtype == "e2m1":
            a = e2m1_codes(w.M, w.K, g)
            b = e2m1_codes(w.N, w.K, g)
        else:
            a = fp6_codes(w.M, w.K, g)
            b = fp6_codes(w.N, w.K, g)
        lo, hi = w.scale_exp
        sa = e8m0_scales((w.M, w.K // 32), g, lo, hi)
        sb = e8m0_scales((w.N, w.K // 32), g, lo, hi)
        return {"A": a, "B": b, "SA": sa, "SB": sb}
    dt = TORCH_DTYPES[w.dtype]
    if w.dist == "uniform":
        a, b = uniform(shp_a, g, dt), uniform(shp_b, g, dt)
    else:
        a, b = normal(shp_a, g, w.sigma, dt), normal(shp_b, g, w.sigma, dt)
    return {"A": a, "B": b}


def raw(t: torch.Tensor):
    """The storage of a CPU tensor as a numpy array of unsigned integers
    (uint16 for 16-bit formats, uint8 for bytes), for the oracle."""
    t = t.contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype in (torch.uint8, torch.float8_e4m3fn, torch.float8_e8m0fnu):
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"no raw view for {t.dtype}")
