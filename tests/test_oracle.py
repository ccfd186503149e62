"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Each check is chosen so that a plausible slip in the oracle -- a wrong
decoder bit, a dropped K term, a transposed or swapped operand, a scale
applied to the wrong block -- fails at least one of them:

* decoders: every bit pattern of float16, bfloat16, E4M3 and E8M0 against
  torch's own casts to float64 (an independent library routine);
* brute force: exact rational sums (fractions.Fraction) on tiny random shapes;
* identity / permutation operands: the output is a transposed or permuted
  copy of an input, bit for bit;
* all-ones operands: the closed form K (and its MX analogue with scales);
* quarter-integer operands (the input structure of the 16x8x32 example on the
  "mma.sync" page, Examples): exact integer arithmetic;
* invariants: transpose symmetry, power-of-two linearity, batch slices, MX
  with unit scales equals the plain E4M3 product, uniform scale shifts;
* E2M1 (MXFP4): the format's sixteen values as the OCP specification lists
  them, the nibble order of a hand-packed byte, every value re-encoded by
  torch's own E4M3 cast decoding the same, and the MXFP4 product equal to the
  MXFP8 product of the same values (E2M1 is a subset of E4M3), plus brute
  force;
* FP6 (MXFP6, E2M3 and E3M2): the value sets as the OCP specification lays
  them out (ranges and steps, not recomputed from bit fields), the bit order
  of a hand-packed three-byte group, every value re-encoded by torch's E4M3
  cast decoding the same (both formats are subsets of E4M3), the MXFP6
  product equal to the MXFP8 product of the same values, and brute force;
* NVFP4 (E2M1 with an E4M3 scale per 16 and an fp32 scale per tensor): with
  power-of-two block scales equal across each 32-block and unit tensor scales
  it is the MXFP4 product of the same powers; power-of-two tensor scales
  scale exactly; brute force with the block scales decoded by torch's E4M3;
  a scale read per 32 instead of per 16 breaks the pins;
* operand arrangements and leading dimensions: every row-/column-major pair,
  stored through torch's own transposes inside NaN-padded rows, equals the
  pinned TN product bit for bit (a swapped index or an ignored leading
  dimension reads a NaN or a wrong element);
* MXFP8 operands in either arrangement: every row-/column-major pair with
  E4M3 elements stored through torch's transposes inside rows padded with
  the E4M3 NaN byte, each element scaled by the block of its logical row of
  A (column of B), equals the pinned TN MX product bit for bit; a wrong
  order flag or A's scales applied to B break it;
* the epilogue's per-element operations: relu's closed form; x * Phi(x)
  against printed standard normal table values; op(x) - op(-x) = x for the
  odd-part forms (gelu, silu); silu at +-ln 3, where the logistic function is
  3/4 and 1/4; the tanh form of gelu within its known 5e-4 of the erf form,
  and both approaching x and 0 in the tails.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from tensor_core_matrix_amd import inputs as inp

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _same(x, y):
    """Bitwise-equal float64 arrays, NaN matching NaN."""
    x, y = np.asarray(x, np.float64), np.asarray(y, np.float64)
    return x.shape == y.shape and bool(np.all((x == y) | (np.isnan(x) & np.isnan(y))))


def _e2m1_to_e4m3(codes_packed: np.ndarray) -> np.ndarray:
    """E4M3 bytes holding the same values as packed E2M1 pairs, encoded by
    torch's float8 cast (every E2M1 value is exactly an E4M3 value)."""
    v = orc.decode(orc.E2M1, codes_packed)
    return torch.from_numpy(v).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------- decoders
def test_decode_f16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    assert _same(orc.decode(orc.F16, bits), want)


def test_decode_bf16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert _same(orc.decode(orc.BF16, bits), want)


def test_decode_e4m3_all_patterns():
    bits = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(bits).view(torch.float8_e4m3fn).double().numpy()
    got = orc.decode(orc.E4M3, bits)
    assert _same(got, want)
    assert np.nanmax(got) == 448.0 and np.isnan(got).sum() == 2  # 0x7F, 0xFF


def test_decode_e2m1_all_codes_and_nibble_order():
    # OCP MX E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7 (sign
    # in bit 3), listed here as the specification's table, not recomputed
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    codes = np.arange(16, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    got = orc.decode(orc.E2M1, packed)
    assert list(got[:8]) == table and list(-got[8:]) == table
    assert np.signbit(got[8])  # code 8 is -0
    # byte 0x21 holds element 0 = code 1 (0.5) in its low nibble, element 1 =
    # code 2 (1.0) in its high nibble; 0xF7: 6.0, then code 15 = -6.0
    assert list(orc.decode(orc.E2M1, np.array([0x21, 0xF7], np.uint8))) == [0.5, 1.0, 6.0, -6.0]
    # each value, re-encoded by torch's E4M3 cast, decodes identically
    assert _same(orc.decode(orc.E4M3, _e2m1_to_e4m3(packed)), got)


def _fp6_table(fmt):
    """Non-negative values of the 32 positive FP6 codes as the OCP MX
    specification lays them out: subnormals, then each binade's steps."""
    if fmt == "e2m3":   # subnormals k/8; binades [1,2) step 1/8, [2,4) 1/4, [4,8) 1/2
        return ([Fraction(k, 8) for k in range(8)] + [1 + Fraction(k, 8) for k in range(8)]
                + [2 + Fraction(k, 4) for k in range(8)] + [4 + Fraction(k, 2) for k in range(8)])
    # e3m2: subnormals k/16; binades from 1/4 to 16, four steps each (max 28)
    vals = [Fraction(k, 16) for k in range(4)]
    for e in range(-2, 5):
        vals += [Fraction(2) ** e * (1 + Fraction(k, 4)) for k in range(4)]
    return vals


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_decode_fp6_all_codes_and_bit_order(fmt):
    dt = orc.DTYPE_NAMES[fmt]
    table = _fp6_table(fmt)
    assert len(table) == 32 and table == sorted(table)
    assert max(table) == (Fraction(15, 2) if fmt == "e2m3" else 28)
    codes = torch.arange(64, dtype=torch.int32).reshape(1, 64)
    got = orc.decode(dt, inp.raw(inp.pack_fp6(codes)))[0]
    assert [Fraction(v) for v in got[:32]] == table
    assert [Fraction(-v) for v in got[32:]] == table and np.signbit(got[32])
    # codes 1, 2, 3, 4 packed by hand: bits 0-5 = 1, 6-11 = 2, 12-17 = 3,
    # 18-23 = 4 -> bytes 0x81, 0x30, 0x10
    hand = np.array([[0x81, 0x30, 0x10]], np.uint8)
    assert list(orc.decode(dt, hand)[0]) == [float(table[c]) for c in (1, 2, 3, 4)]
    assert np.array_equal(inp.raw(inp.pack_fp6(torch.tensor([[1, 2, 3, 4]]))), hand)
    # every value, re-encoded by torch's E4M3 cast, decodes identically
    e4 = torch.from_numpy(got).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert _same(orc.decode(orc.E4M3, e4), got)


def _fp6_to_e4m3(dt, packed: np.ndarray) -> np.ndarray:
    v = orc.decode(dt, packed)
    return torch.from_numpy(v).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_mxfp6_equals_mxfp8_of_the_same_values(fmt):
    dt = orc.DTYPE_NAMES[fmt]
    M, N, K = 9, 7, 128
    g = inp.generator(49)
    a, b = inp.fp6_codes(M, K, g), inp.fp6_codes(N, K, g)
    sa, sb = inp.e8m0_scales((M, K // 32), g), inp.e8m0_scales((N, K // 32), g)
    r6, s6 = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), dtype=dt)
    r8, s8 = orc.gemm_mx(_fp6_to_e4m3(dt, inp.raw(a)), _fp6_to_e4m3(dt, inp.raw(b)),
                         inp.raw(sa), inp.raw(sb))
    assert _same(r6, r8) and _same(s6, s8)
    ii, jj = np.array([0, 8, 4]), np.array([6, 0, 3])
    re, se = orc.entries(dt, inp.raw(a), inp.raw(b), ii, jj, sa=inp.raw(sa), sb=inp.raw(sb))
    assert _same(re, r6[ii, jj]) and _same(se, s6[ii, jj])


@pytest.mark.parametrize("shape", [(1, 1, 32), (3, 4, 64)])
def test_brute_force_mxfp6(shape):
    M, N, K = shape
    g = inp.generator(50 + K)
    codes_a = torch.randint(0, 64, (M, K), generator=g, dtype=torch.int32)
    codes_b = torch.randint(0, 64, (N, K), generator=g, dtype=torch.int32)
    sa = inp.e8m0_scales((M, K // 32), g, -6, 6)
    sb = inp.e8m0_scales((N, K // 32), g, -6, 6)
    table = _fp6_table("e3m2")
    val = lambda c: -table[c - 32] if c >= 32 else table[c]   # values from the codes
    ref, _ = orc.gemm_mx(inp.raw(inp.pack_fp6(codes_a)), inp.raw(inp.pack_fp6(codes_b)),
                         inp.raw(sa), inp.raw(sb), dtype=orc.E3M2)
    ea = sa.numpy().astype(np.int64) - 127
    eb = sb.numpy().astype(np.int64) - 127
    for i in range(M):
        for j in range(N):
            ex = sum((val(int(codes_a[i, k])) * Fraction(2) ** int(ea[i, k // 32])
                      * val(int(codes_b[j, k])) * Fraction(2) ** int(eb[j, k // 32])
                      for k in range(K)), Fraction(0))
            assert Fraction(ref[i, j]) == ex


def _nv4_case(M, N, K, seed):
    g = inp.generator(seed)
    return (inp.e2m1_codes(M, K, g), inp.e2m1_codes(N, K, g),
            inp.e4m3_scales((M, K // 16), g), inp.e4m3_scales((N, K // 16), g))


def test_nvfp4_power_of_two_scales_equal_mxfp4():
    M, N, K = 9, 7, 128
    g = inp.generator(51)
    a, b = inp.e2m1_codes(M, K, g), inp.e2m1_codes(N, K, g)
    ea = torch.randint(-5, 6, (M, K // 32), generator=g)
    eb = torch.randint(-5, 6, (N, K // 32), generator=g)
    # E4M3 2^e: exponent field e + 7, mantissa 0; each 32-block's two halves alike
    sa4 = ((ea + 7) << 3).repeat_interleave(2, dim=1).to(torch.uint8)
    sb4 = ((eb + 7) << 3).repeat_interleave(2, dim=1).to(torch.uint8)
    ref, s = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa4), inp.raw(sb4), 1.0, 1.0)
    mx, ms = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw((ea + 127).to(torch.uint8)),
                         inp.raw((eb + 127).to(torch.uint8)), dtype=orc.E2M1)
    assert _same(ref, mx) and _same(s, ms)
    # power-of-two tensor scales scale exactly; others to within fp64 rounding
    r2, _ = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa4), inp.raw(sb4), 4.0, 0.125)
    assert _same(r2, 0.5 * ref)
    r3, _ = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa4), inp.raw(sb4), 0.3, 1.0)
    assert np.all(np.abs(r3 - 0.3 * ref) <= 1e-14 * 0.3 * s)   # relative to sum |terms|


@pytest.mark.parametrize("shape", [(1, 1, 32), (3, 4, 64)])
def test_brute_force_nvfp4(shape):
    M, N, K = shape
    a, b, sa, sb = _nv4_case(M, N, K, 52 + K)
    ref, _ = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), 0.75, -2.0)
    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
           Fraction(4), Fraction(6)]

    def val(packed, r, k):
        byte = int(packed[r, k // 2])
        c = (byte >> 4) if k % 2 else (byte & 15)
        return -mag[c & 7] if c & 8 else mag[c & 7]

    # block scales decoded by torch's own E4M3 type, not by the oracle
    fa = sa.view(torch.float8_e4m3fn).double().numpy()
    fb = sb.view(torch.float8_e4m3fn).double().numpy()
    an, bn = a.numpy(), b.numpy()
    for i in range(M):
        for j in range(N):
            ex = sum((val(an, i, k) * Fraction(fa[i, k // 16]) * val(bn, j, k) * Fraction(fb[j, k // 16])
                      for k in range(K)), Fraction(0)) * Fraction(0.75) * Fraction(-2.0)
            assert abs(Fraction(ref[i, j]) - ex) <= Fraction(K * 2.0 ** -52) * abs(ex) + Fraction(2.0 ** -1000)


def test_nvfp4_entries_and_planted_block_size():
    M, N, K = 13, 11, 96
    a, b, sa, sb = _nv4_case(M, N, K, 53)
    ref, s = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), 1.5, 0.5)
    ii, jj = np.array([0, 12, 7]), np.array([10, 0, 4])
    r, ss = orc.entries_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), 1.5, 0.5, ii, jj)
    assert _same(r, ref[ii, jj]) and _same(ss, s[ii, jj])
    # planted on the CPU: one scale per 32 (the even 16-blocks' scale used for
    # both halves) is a different product
    wrong_a = sa[:, 0::2].repeat_interleave(2, dim=1).contiguous()
    wrong_b = sb[:, 0::2].repeat_interleave(2, dim=1).contiguous()
    w, _ = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(wrong_a), inp.raw(wrong_b), 1.5, 0.5)
    assert not _same(w, ref)


def test_decode_e8m0_all_patterns():
    bits = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(bits).view(torch.float8_e8m0fnu).float().double().numpy()
    got = orc.decode(orc.E8M0, bits)
    assert _same(got, want)
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and np.isnan(got[255])


# ------------------------------------------------------------- brute force
def _exact(av, bv):
    """Exact rational A . B^T from float64-representable values."""
    M, K = av.shape
    N = bv.shape[0]
    out = [[sum((Fraction(float(av[i, k])) * Fraction(float(bv[j, k])) for k in range(K)),
                Fraction(0)) for j in range(N)] for i in range(M)]
    return out


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (8, 2, 16), (5, 8, 3)])
def test_brute_force_plain(dt, shape):
    M, N, K = shape
    g = inp.generator(11 + M * 100 + N * 10 + K)
    tdt = inp.TORCH_DTYPES[dt]
    a = inp.normal((M, K), g, 3.0, tdt)
    b = inp.normal((N, K), g, 3.0, tdt)
    ref, s = orc.gemm_tn(orc.DTYPE_NAMES[dt], inp.raw(a), inp.raw(b))
    ex = _exact(a.double().numpy(), b.double().numpy())
    for i in range(M):
        for j in range(N):
            assert abs(Fraction(ref[i, j]) - ex[i][j]) <= Fraction(K * 2.0 ** -52) * Fraction(s[i, j])
    # abssum is the exact |.| sum up to the same rounding
    absx = _exact(np.abs(a.double().numpy()), np.abs(b.double().numpy()))
    for i in range(M):
        for j in range(N):
            assert abs(Fraction(s[i, j]) - absx[i][j]) <= Fraction(K * 2.0 ** -52) * absx[i][j]


@pytest.mark.parametrize("shape", [(1, 1, 32), (3, 4, 64), (4, 2, 96)])
def test_brute_force_mx(shape):
    M, N, K = shape
    g = inp.generator(5 + K)
    a = inp.e4m3_normal((M, K), g)
    b = inp.e4m3_normal((N, K), g)
    sa = inp.e8m0_scales((M, K // 32), g, -6, 6)
    sb = inp.e8m0_scales((N, K // 32), g, -6, 6)
    ref, s = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb))
    av = a.view(torch.float8_e4m3fn).double().numpy()
    bv = b.view(torch.float8_e4m3fn).double().numpy()
    ea = sa.numpy().astype(np.int64) - 127
    eb = sb.numpy().astype(np.int64) - 127
    for i in range(M):
        for j in range(N):
            ex = sum((Fraction(float(av[i, k])) * Fraction(2) ** int(ea[i, k // 32])
                      * Fraction(float(bv[j, k])) * Fraction(2) ** int(eb[j, k // 32])
                      for k in range(K)), Fraction(0))
            assert abs(Fraction(ref[i, j]) - ex) <= Fraction(K * 2.0 ** -52) * Fraction(s[i, j])


@pytest.mark.parametrize("shape", [(1, 1, 32), (3, 4, 64), (2, 3, 96)])
def test_brute_force_mxfp4(shape):
    M, N, K = shape
    g = inp.generator(40 + K)
    a = inp.e2m1_codes(M, K, g)
    b = inp.e2m1_codes(N, K, g)
    sa = inp.e8m0_scales((M, K // 32), g, -6, 6)
    sb = inp.e8m0_scales((N, K // 32), g, -6, 6)
    ref, s = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), dtype=orc.E2M1)
    # element values straight from the specification's table and the
    # low-nibble-first packing, independent of the oracle's decoder
    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
           Fraction(4), Fraction(6)]

    def val(packed, r, k):
        byte = int(packed[r, k // 2])
        c = (byte >> 4) if k % 2 else (byte & 15)
        return -mag[c & 7] if c & 8 else mag[c & 7]

    an, bn = a.numpy(), b.numpy()
    ea = sa.numpy().astype(np.int64) - 127
    eb = sb.numpy().astype(np.int64) - 127
    for i in range(M):
        for j in range(N):
            ex = sum((val(an, i, k) * Fraction(2) ** int(ea[i, k // 32])
                      * val(bn, j, k) * Fraction(2) ** int(eb[j, k // 32])
                      for k in range(K)), Fraction(0))
            assert Fraction(ref[i, j]) == ex  # every term and partial sum is exact in fp64


def test_mxfp4_equals_mxfp8_of_the_same_values():
    M, N, K = 9, 7, 128
    g = inp.generator(44)
    a = inp.e2m1_codes(M, K, g)
    b = inp.e2m1_codes(N, K, g)
    sa = inp.e8m0_scales((M, K // 32), g)
    sb = inp.e8m0_scales((N, K // 32), g)
    r4, s4 = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), dtype=orc.E2M1)
    r8, s8 = orc.gemm_mx(_e2m1_to_e4m3(inp.raw(a)), _e2m1_to_e4m3(inp.raw(b)), inp.raw(sa),
                         inp.raw(sb))
    assert _same(r4, r8) and _same(s4, s8)
    ii, jj = np.array([0, 8, 4]), np.array([6, 0, 3])
    re, se = orc.entries(orc.E2M1, inp.raw(a), inp.raw(b), ii, jj, sa=inp.raw(sa),
                         sb=inp.raw(sb))
    assert _same(re, r4[ii, jj]) and _same(se, s4[ii, jj])


# ------------------------------------------------- identity / permutation
def test_identity_left_gives_transpose_of_b():
    K, N = 48, 40
    g = inp.generator(21)
    a = torch.eye(K, dtype=torch.bfloat16)
    b = inp.normal((N, K), g, 1.0, torch.bfloat16)
    ref, _ = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    assert _same(ref, b.double().numpy().T)  # Out[i, j] = B[j, i]


def test_identity_right_gives_a():
    M, K = 33, 24
    g = inp.generator(22)
    a = inp.normal((M, K), g, 1.0, torch.float16)
    b = torch.eye(K, dtype=torch.float16)
    ref, _ = orc.gemm_tn(orc.F16, inp.raw(a), inp.raw(b))
    assert _same(ref, a.double().numpy())


def test_permutation_permutes_columns():
    M, K = 17, 32
    g = inp.generator(23)
    a = inp.normal((M, K), g, 1.0, torch.bfloat16)
    perm = torch.randperm(K, generator=g)
    b = torch.zeros(K, K, dtype=torch.bfloat16)
    b[torch.arange(K), perm] = 1  # B[j, perm[j]] = 1
    ref, _ = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    assert _same(ref, a.double().numpy()[:, perm.numpy()])  # Out[i, j] = A[i, perm[j]]


# ------------------------------------------------------------ closed forms
@pytest.mark.parametrize("K", [1, 64, 1000])
def test_all_ones_is_k(K):
    a = torch.ones(5, K, dtype=torch.bfloat16)
    b = torch.ones(7, K, dtype=torch.bfloat16)
    ref, s = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    assert np.all(ref == K) and np.all(s == K)


def test_all_ones_mx_closed_form():
    M, N, K = 6, 5, 128
    g = inp.generator(24)
    one = 0x38  # E4M3 1.0: exponent field 7 (bias 7), mantissa 0
    a = torch.full((M, K), one, dtype=torch.uint8)
    b = torch.full((N, K), one, dtype=torch.uint8)
    sa = inp.e8m0_scales((M, K // 32), g, -4, 4)
    sb = inp.e8m0_scales((N, K // 32), g, -4, 4)
    ref, _ = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb))
    ea = sa.numpy().astype(np.int64) - 127
    eb = sb.numpy().astype(np.int64) - 127
    want = np.array([[sum(32 * 2.0 ** (ea[i, q] + eb[j, q]) for q in range(K // 32))
                      for j in range(N)] for i in range(M)])
    assert _same(ref, want)


# -------------------------------------------------------- quarter integers
def test_quarter_integer_page_example_exact():
    """The 16x8x32 example's input recipe (numpy default_rng(0), integers in
    [-4, 5) divided by 4, float16): every partial sum is a multiple of 1/16, so
    the exact result is an integer product divided by 16."""
    rng = np.random.default_rng(0)
    ai = rng.integers(-4, 5, (16, 32))
    bi = rng.integers(-4, 5, (8, 32))
    a = (ai / 4).astype("float16")
    b = (bi / 4).astype("float16")
    ref, _ = orc.gemm_tn(orc.F16, a.view("uint16"), b.view("uint16"))
    assert _same(ref, (ai @ bi.T) / 16.0)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_quarter_integer_tile_exact(dt):
    M, N, K = 128, 64, 64
    g = inp.generator(25)
    a = inp.quarter_integers((M, K), g, inp.TORCH_DTYPES[dt])
    b = inp.quarter_integers((N, K), g, inp.TORCH_DTYPES[dt])
    ai = (a.float() * 4).round().long().numpy()
    bi = (b.float() * 4).round().long().numpy()
    ref, _ = orc.gemm_tn(orc.DTYPE_NAMES[dt], inp.raw(a), inp.raw(b))
    assert _same(ref, (ai @ bi.T) / 16.0)


# --------------------------------------------------------------- invariants
def test_transpose_symmetry_and_linearity():
    g = inp.generator(26)
    a = inp.normal((19, 40), g, 1.0, torch.bfloat16)
    b = inp.normal((23, 40), g, 1.0, torch.bfloat16)
    r_ab, _ = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    r_ba, _ = orc.gemm_tn(orc.BF16, inp.raw(b), inp.raw(a))
    assert _same(r_ab, r_ba.T)
    r_2a, _ = orc.gemm_tn(orc.BF16, inp.raw(a * 2), inp.raw(b))
    assert _same(r_2a, 2 * r_ab)


def test_batch_slices_equal_single_problems():
    g = inp.generator(27)
    a = inp.uniform((3, 9, 16), g, torch.bfloat16)
    b = inp.uniform((3, 11, 16), g, torch.bfloat16)
    rb, sb = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    for p in range(3):
        r1, s1 = orc.gemm_tn(orc.BF16, inp.raw(a[p]), inp.raw(b[p]))
        assert _same(rb[p], r1) and _same(sb[p], s1)


def test_mx_unit_scales_equal_plain_e4m3_and_shift():
    M, N, K = 7, 6, 64
    g = inp.generator(28)
    a = inp.e4m3_normal((M, K), g)
    b = inp.e4m3_normal((N, K), g)
    unit_a = torch.full((M, K // 32), 127, dtype=torch.uint8)
    unit_b = torch.full((N, K // 32), 127, dtype=torch.uint8)
    r_mx, _ = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(unit_a), inp.raw(unit_b))
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    r_plain, _ = orc.entries(orc.E4M3, inp.raw(a), inp.raw(b), ii.ravel(), jj.ravel())
    assert _same(r_mx.ravel(), r_plain)
    # shifting every A scale by +3 and every B scale by -1 multiplies by 2^2
    r_sh, _ = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(unit_a + 3), inp.raw(unit_b - 1))
    assert _same(r_sh, 4 * r_mx)
    # a scale change in one block touches only that block's terms
    sa = unit_a.clone()
    sa[2, 1] = 127 + 5
    r_blk, _ = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(unit_b))
    av = a.view(torch.float8_e4m3fn).double().numpy()
    bv = b.view(torch.float8_e4m3fn).double().numpy()
    delta = (2.0 ** 5 - 1) * (av[2, 32:64] @ bv[:, 32:64].T)
    assert np.allclose(r_blk[2] - r_mx[2], delta, rtol=0, atol=1e-12)
    assert _same(np.delete(r_blk, 2, 0), np.delete(r_mx, 2, 0))


def test_entries_match_full_product():
    g = inp.generator(29)
    a = inp.normal((2, 13, 24), g, 1.0, torch.float16)
    b = inp.normal((2, 9, 24), g, 1.0, torch.float16)
    full, fs = orc.gemm_tn(orc.F16, inp.raw(a), inp.raw(b))
    bb = np.array([0, 1, 1, 0])
    ii = np.array([0, 12, 5, 7])
    jj = np.array([8, 0, 3, 4])
    r, s = orc.entries(orc.F16, inp.raw(a), inp.raw(b), ii, jj, bb=bb)
    assert _same(r, full[bb, ii, jj]) and _same(s, fs[bb, ii, jj])


def test_nan_inputs_propagate():
    a = torch.ones(2, 8, dtype=torch.bfloat16)
    a[1, 3] = float("nan")
    b = torch.ones(3, 8, dtype=torch.bfloat16)
    ref, _ = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    assert np.all(ref[0] == 8) and np.all(np.isnan(ref[1]))


# -------------------------------------------- planted mistakes are caught
def test_planted_mistakes_fail_the_pins():
    """Planted on the CPU: reading B as K x N (A . B instead of A . B^T) or a
    dropped K term must break the permutation and closed-form pins above."""
    M, K = 17, 32
    g = inp.generator(30)
    a = inp.normal((M, K), g, 1.0, torch.bfloat16)
    perm = torch.randperm(K, generator=g)
    b = torch.zeros(K, K, dtype=torch.bfloat16)
    b[torch.arange(K), perm] = 1
    want = a.double().numpy()[:, perm.numpy()]
    untransposed, _ = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b.T.contiguous()))  # A . B
    assert not _same(untransposed, want)
    dropped, _ = orc.gemm_tn(orc.BF16, inp.raw(torch.ones(3, 63, dtype=torch.bfloat16)),
                             inp.raw(torch.ones(4, 63, dtype=torch.bfloat16)))
    assert not np.all(dropped == 64)


# --------------------------------- arrangements and leading dimensions
def _in_nan_rows(x: torch.Tensor, ld: int) -> torch.Tensor:
    """x (rows x c) in the first c columns of a rows x ld array whose other
    elements are NaN: row-major storage of x with leading dimension ld."""
    out = torch.full((x.shape[0], ld), float("nan"), dtype=x.dtype)
    out[:, : x.shape[1]] = x
    return out


def _stored(a, b, a_order, b_order, pad):
    """Storage and leading dimensions of logical A = a (M x K) and B = b^T
    (K x N) in the given orders, made with torch's transposes."""
    ast = a if a_order == orc.ROW_MAJOR else a.T      # column-major A: rows of A^T
    bst = b.T if b_order == orc.ROW_MAJOR else b      # column-major B: rows of B^T = b
    lda, ldb = ast.shape[1] + pad, bst.shape[1] + pad
    return _in_nan_rows(ast, lda), lda, _in_nan_rows(bst, ldb), ldb


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("a_order", [0, 1])
@pytest.mark.parametrize("b_order", [0, 1])
@pytest.mark.parametrize("pad", [0, 5])
def test_arrangements_equal_tn_product(dt, a_order, b_order, pad):
    M, N, K = 13, 11, 24
    g = inp.generator(46 + a_order + 2 * b_order)
    tdt = inp.TORCH_DTYPES[dt]
    a = inp.normal((M, K), g, 1.0, tdt)
    b = inp.normal((N, K), g, 1.0, tdt)
    want, ws = orc.gemm_tn(orc.DTYPE_NAMES[dt], inp.raw(a), inp.raw(b))
    ast, lda, bst, ldb = _stored(a, b, a_order, b_order, pad)
    got, gs = orc.gemm_ld(orc.DTYPE_NAMES[dt], inp.raw(ast), a_order, lda, inp.raw(bst),
                          b_order, ldb, M, N, K)
    assert _same(got, want) and _same(gs, ws)
    ii, jj = np.array([0, 12, 7]), np.array([10, 0, 4])
    r, s = orc.entries_ld(orc.DTYPE_NAMES[dt], inp.raw(ast), a_order, lda, inp.raw(bst), b_order,
                          ldb, M, N, K, ii, jj)
    assert _same(r, want[ii, jj]) and _same(s, ws[ii, jj])


def test_arrangement_exact_against_numpy_matmul():
    """Small-integer operands: the product is exact in fp64, so it must equal
    numpy's matmul of the logical matrices (column-major A, row-major B)."""
    M, N, K = 6, 9, 40
    g = inp.generator(47)
    a = torch.randint(-8, 9, (K, M), generator=g).to(torch.bfloat16)   # storage of A^T
    b = torch.randint(-8, 9, (K, N), generator=g).to(torch.bfloat16)   # storage of B
    got, _ = orc.gemm_ld(orc.BF16, inp.raw(a), orc.COL_MAJOR, M, inp.raw(b), orc.ROW_MAJOR, N,
                         M, N, K)
    assert np.array_equal(got, a.double().numpy().T @ b.double().numpy())


def test_arrangement_validation():
    z = np.zeros(64, np.uint16)
    with pytest.raises(ValueError):   # row-major A needs lda >= K
        orc.gemm_ld(orc.BF16, z, orc.ROW_MAJOR, 3, z, orc.COL_MAJOR, 4, 2, 2, 4)
    with pytest.raises(ValueError):   # column-major A needs lda >= M
        orc.gemm_ld(orc.BF16, z, orc.COL_MAJOR, 1, z, orc.COL_MAJOR, 4, 2, 2, 4)
    with pytest.raises(ValueError):   # storage too small for the leading dimension
        orc.gemm_ld(orc.BF16, z, orc.ROW_MAJOR, 70, z, orc.COL_MAJOR, 4, 2, 2, 4)
    with pytest.raises(ValueError):   # unknown order
        orc.gemm_ld(orc.BF16, z, 2, 4, z, orc.COL_MAJOR, 4, 2, 2, 4)


def test_planted_arrangement_mistakes_fail_the_pin():
    """Planted on the CPU: reading column-major storage as row-major, or
    stepping rows by the column count instead of the leading dimension, must
    break the equality with the TN product."""
    M = N = K = 16
    g = inp.generator(48)
    a = inp.normal((M, K), g, 1.0, torch.bfloat16)
    b = inp.normal((N, K), g, 1.0, torch.bfloat16)
    want, _ = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    ast, lda, bst, ldb = _stored(a, b, orc.COL_MAJOR, orc.ROW_MAJOR, 3)
    wrong_order, _ = orc.gemm_ld(orc.BF16, inp.raw(ast), orc.ROW_MAJOR, lda, inp.raw(bst),
                                 orc.ROW_MAJOR, ldb, M, N, K)
    assert not _same(wrong_order, want)
    wrong_ld, _ = orc.gemm_ld(orc.BF16, inp.raw(ast), orc.COL_MAJOR, M, inp.raw(bst),
                              orc.ROW_MAJOR, ldb, M, N, K)
    assert not _same(wrong_ld, want)


def _stored_bytes(a, b, a_order, b_order, pad):
    """As _stored, for E4M3 operands held as bytes: the padding is the E4M3
    NaN byte 0x7F."""
    ast = a if a_order == orc.ROW_MAJOR else a.T
    bst = b.T if b_order == orc.ROW_MAJOR else b
    lda, ldb = ast.shape[1] + pad, bst.shape[1] + pad
    def rows(x, ld):
        out = torch.full((x.shape[0], ld), 0x7F, dtype=torch.uint8)
        out[:, : x.shape[1]] = x
        return out
    return rows(ast, lda), lda, rows(bst, ldb), ldb


@pytest.mark.parametrize("a_order", [0, 1])
@pytest.mark.parametrize("b_order", [0, 1])
@pytest.mark.parametrize("pad", [0, 7])
def test_mx_arrangements_equal_tn_mx_product(a_order, b_order, pad):
    """MXFP8 in either arrangement: the E4M3 elements found through the
    arrangement, each scaled by the block of its logical row of A (column of
    B), equal the pinned TN MX product bit for bit."""
    M, N, K = 13, 11, 96
    g = inp.generator(49 + a_order + 2 * b_order)
    a = inp.raw(inp.e4m3_normal((M, K), g))
    b = inp.raw(inp.e4m3_normal((N, K), g))
    sa, sb = inp.e8m0_scales((M, K // 32), g), inp.e8m0_scales((N, K // 32), g)
    want, ws = orc.gemm_mx(a, b, inp.raw(sa), inp.raw(sb))
    ast, lda, bst, ldb = _stored_bytes(torch.from_numpy(a), torch.from_numpy(b), a_order, b_order,
                                       pad)
    got, gs = orc.gemm_mx_ld(ast.numpy(), a_order, lda, bst.numpy(), b_order, ldb, inp.raw(sa),
                             inp.raw(sb), M, N, K)
    assert _same(got, want) and _same(gs, ws)
    ii, jj = np.array([0, 12, 7]), np.array([10, 0, 4])
    r, rs = orc.entries_mx_ld(ast.numpy(), a_order, lda, bst.numpy(), b_order, ldb, inp.raw(sa),
                              inp.raw(sb), M, N, K, ii, jj)
    assert _same(r, want[ii, jj]) and _same(rs, ws[ii, jj])


def test_mx_arrangement_planted_mistakes_fail_the_pin():
    """Planted on the CPU: the order flag or leading dimension read wrongly,
    or A's scales applied to B, must break the equality."""
    M = N = 32
    K = 64
    g = inp.generator(50)
    a = inp.raw(inp.e4m3_normal((M, K), g))
    b = inp.raw(inp.e4m3_normal((N, K), g))
    sa, sb = inp.raw(inp.e8m0_scales((M, K // 32), g)), inp.raw(inp.e8m0_scales((N, K // 32), g))
    want, _ = orc.gemm_mx(a, b, sa, sb)
    ast, lda, bst, ldb = _stored_bytes(torch.from_numpy(a), torch.from_numpy(b), orc.COL_MAJOR,
                                       orc.ROW_MAJOR, 0)
    ast, bst = ast.numpy(), bst.numpy()
    ok, _ = orc.gemm_mx_ld(ast, orc.COL_MAJOR, lda, bst, orc.ROW_MAJOR, ldb, sa, sb, M, N, K)
    assert _same(ok, want)
    bad, _ = orc.gemm_mx_ld(ast, orc.ROW_MAJOR, K, bst, orc.ROW_MAJOR, ldb, sa, sb, M, N, K)
    assert not _same(bad, want)
    bad, _ = orc.gemm_mx_ld(ast, orc.COL_MAJOR, lda, bst, orc.ROW_MAJOR, ldb, sb, sa, M, N, K)
    assert not _same(bad, want)


def test_mx_arrangement_validation():
    z8 = np.zeros(4096, np.uint8)
    s = np.zeros((4, 1), np.uint8)
    with pytest.raises(ValueError):   # K not a multiple of 32
        orc.gemm_mx_ld(z8, orc.ROW_MAJOR, 48, z8, orc.COL_MAJOR, 48, s, s, 4, 4, 48)
    with pytest.raises(ValueError):   # column-major A needs lda >= M
        orc.gemm_mx_ld(z8, orc.COL_MAJOR, 2, z8, orc.COL_MAJOR, 32, s, s, 4, 4, 32)
    with pytest.raises(ValueError):   # scale tensor of the wrong shape
        orc.gemm_mx_ld(z8, orc.ROW_MAJOR, 32, z8, orc.COL_MAJOR, 32, s[:3], s, 4, 4, 32)


# --------------------------------------------- per-element epilogue ops
def test_op_relu_and_identity_closed_form():
    x = np.array([-3.5, -1e-30, 0.0, 1e-30, 2.25, 7.0])
    assert np.array_equal(orc.apply_op(orc.OPS["identity"], x), x)
    assert np.array_equal(orc.apply_op(orc.OPS["relu"], x), [0, 0, 0, 1e-30, 2.25, 7.0])


def test_op_gelu_erf_is_x_times_normal_cdf():
    # standard normal distribution function Phi at 1, 2, -1 and 0.5, as
    # printed in statistical tables
    phi = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, -1.0: 0.15865525393145707,
           0.5: 0.6914624612740131}
    x = np.array(list(phi))
    got = orc.apply_op(orc.OPS["gelu_erf"], x)
    assert np.allclose(got, x * np.array(list(phi.values())), rtol=1e-14, atol=0)
    # deep in the negative tail erfc keeps full relative accuracy:
    # Phi(-10) = 7.619853024160527e-24
    assert abs(orc.apply_op(3, np.array([-10.0]))[0] / (-10 * 7.619853024160527e-24) - 1) < 1e-12


@pytest.mark.parametrize("name", ["gelu_tanh", "gelu_erf", "silu"])
def test_op_odd_part_identity(name):
    """x/2 (1 + f(x)) with f odd gives op(x) - op(-x) = x."""
    x = np.linspace(-9, 9, 181)
    d = orc.apply_op(orc.OPS[name], x) - orc.apply_op(orc.OPS[name], -x)
    assert np.allclose(d, x, rtol=0, atol=1e-13)


def test_op_silu_at_log3():
    # logistic(ln 3) = 3/4, logistic(-ln 3) = 1/4
    l3 = np.log(3.0)
    got = orc.apply_op(orc.OPS["silu"], np.array([l3, -l3, 0.0]))
    assert np.allclose(got, [0.75 * l3, -0.25 * l3, 0.0], rtol=1e-15, atol=0)


def test_op_gelu_tanh_approximates_gelu_erf():
    x = np.linspace(-8, 8, 3201)
    t = orc.apply_op(orc.OPS["gelu_tanh"], x)
    e = orc.apply_op(orc.OPS["gelu_erf"], x)
    err = np.abs(t - e)
    assert err.max() < 5e-4 and err.max() > 1e-5    # the known quality of the tanh form
    assert np.allclose(t[-1], 8.0, atol=1e-12) and abs(t[0]) < 1e-12
    assert orc.apply_op(2, np.array([0.0]))[0] == 0.0


def test_planted_op_mistakes_fail_the_pins():
    """Planted on the CPU: gelu with erf(x) in place of erf(x/sqrt 2), and the
    tanh form without its cubic term, miss the table value and the 5e-4
    agreement."""
    from math import erf, tanh, sqrt, pi
    wrong = 0.5 * 1.0 * (1 + erf(1.0))
    assert abs(wrong - 0.8413447460685429) > 1e-3
    x = np.linspace(-8, 8, 3201)
    no_cube = 0.5 * x * (1 + np.tanh(sqrt(2 / pi) * x))
    assert np.abs(no_cube - orc.apply_op(3, x)).max() > 5e-4


def test_check_op_rule():
    x = np.array([-2.0, -0.5, 0.0, 0.5, 3.0])
    y = orc.apply_op(orc.OPS["gelu_erf"], x)
    ok, worst, nbad = orc.check_op(y, x, 3, 1.0, np.ones(5), np.zeros(5), "f32")
    assert ok and worst == 0.0
    ok, _, nbad = orc.check_op(y + 1e-3, x, 3, 1.0, np.ones(5), np.zeros(5), "f32")
    assert not ok and nbad == 5
    ok, _, _ = orc.check_op(np.array([np.nan]), np.array([1.0]), 1, 1.0, np.ones(1), np.zeros(1),
                            "f32")
    assert not ok


# ----------------------------------------------------- axpby epilogue
def test_axpby_pins():
    g = inp.generator(45)
    M, N, K = 5, 7, 24
    a = inp.normal((M, K), g, 1.0, torch.bfloat16)
    b = inp.normal((N, K), g, 1.0, torch.bfloat16)
    ref, _ = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    # alpha = 1, beta = 0 is the product itself; C may be absent
    assert _same(orc.axpby(1.0, ref), ref)
    # power-of-two alpha scales exactly
    assert _same(orc.axpby(-4.0, ref), -4.0 * ref)
    for name, dt in (("f32", torch.float32), ("bf16", torch.bfloat16), ("f16", torch.float16)):
        c = inp.normal((M, N), g, 3.0, dt)
        cv = c.double().numpy()               # torch's own decode of C
        got = orc.axpby(0.5, ref, -2.0, inp.raw(c), _dt_code(name))
        # 0.5 * ref and -2 * c are exact; their fp64 sum rounds once
        assert np.array_equal(got, 0.5 * ref + (-2.0) * cv)
    # C = the product's own bf16 rounding: alpha + beta = 0 leaves only the
    # rounding error, at most half a bf16 ulp of ref
    cb = torch.from_numpy(ref).to(torch.bfloat16)
    d = orc.axpby(1.0, ref, -1.0, inp.raw(cb), orc.BF16)
    assert np.all(np.abs(d) <= 0.5 * orc.ulp_bf16(ref))
    with pytest.raises(ValueError):
        orc.axpby(1.0, ref, 1.0, None)


def _dt_code(name):
    return orc.DTYPE_NAMES[name]


def test_ulp_f16_matches_bit_spacing():
    g = inp.generator(46)
    v = inp.normal((4096,), g, 100.0, torch.float16).abs()
    v = v[(v > 0) & torch.isfinite(v) & (v < 60000)]
    # the next representable value up: the bit pattern plus one
    up = (v.view(torch.int16) + 1).view(torch.float16).double().numpy()
    assert np.array_equal(up - v.double().numpy(), orc.ulp_f16(v.double().numpy()))
    # subnormal spacing and the smallest normal
    assert orc.ulp_f16(np.array([0.0]))[0] == 2.0 ** -24
    assert orc.ulp_f16(np.array([2.0 ** -14]))[0] == 2.0 ** -24


def test_check_epi_rule():
    exact = np.array([1.0, 1000.0, -3.0])
    ok, _, _ = orc.check_epi(exact + np.array([0.0, 0.5, 0.0]), exact, 1.0, np.zeros(3),
                             np.zeros(3), "f16")
    assert ok                                  # half an f16 ulp at 1000 (ulp 0.5)
    ok, _, nbad = orc.check_epi(exact + np.array([0.0, 1.5, 0.0]), exact, 1.0, np.zeros(3),
                                np.zeros(3), "f16")
    assert not ok and nbad == 1
    ok, _, _ = orc.check_epi(np.array([np.nan, 1000.0, -3.0]), exact, 1.0, np.ones(3),
                             np.zeros(3), "f32")
    assert not ok


# ------------------------------------------------------- comparison rule
def test_ulp_bf16_matches_bit_spacing():
    g = inp.generator(31)
    v = inp.normal((4096,), g, 10.0, torch.bfloat16).abs()
    v = v[(v > 0) & torch.isfinite(v)]
    bits = v.view(torch.int16).numpy().astype(np.int32)
    up = torch.from_numpy((bits + 1).astype(np.int16)).view(torch.bfloat16).double().numpy()
    spacing = up - v.double().numpy()
    assert _same(orc.ulp_bf16(v.double().numpy()), spacing)
    tiny = np.array([0.0, 2.0 ** -130, 2.0 ** -126])
    assert _same(orc.ulp_bf16(tiny), np.full(3, 2.0 ** -133))


def test_check_rule():
    ref = np.array([1.0, -2.0, 0.0, 100.0])
    s = np.array([10.0, 10.0, 0.0, 1000.0])
    ok, worst, nbad = orc.check(ref + np.array([9e-4, -9e-4, 0.0, 0.09]), ref, s, False)
    assert ok and nbad == 0 and worst < 1
    ok, _, nbad = orc.check(ref + np.array([2e-3, 0, 0, 0]), ref, s, False)
    assert not ok and nbad == 1
    ok, _, nbad = orc.check(np.array([1.0, -2.0, np.nan, 100.0]), ref, s, False)
    assert not ok and nbad == 1
    # bf16 output: one ulp of 100 (0.5) is allowed on top of 1e-4 * 1000
    ok, _, _ = orc.check(ref + np.array([0, 0, 0, 0.55]), ref, s, True)
    assert ok
