// The 256 x 256 float16 / bfloat16 product on the 16 x 16 x 32 matrix-core
// instruction of gfx950 (v_mfma_f32_16x16x32_{bf16,f16}).
//
// "Hopper and Blackwell GEMM" (Concept) builds the main loop around the
// largest tensor-core instruction the part offers.  On MI355X the clock is
// set by the power limit, and a matrix core busy with 16 x 16 x 32 products
// draws less power per flop than one busy with 32 x 32 x 16 products (each
// product reads and writes a quarter of the accumulator bytes for half the
// flops): with register operands only, 32 x 32 x 16 products sustain 1.80 GHz
// and 16 x 16 x 32 products 2.04 GHz at the same 99 % matrix-core occupancy.
// This kernel keeps the LDS layout, the copy stream and the tile order of the
// 4-wave 256 x 256 kernel of gemm_kernel.h and changes the product loop:
//
//  * Each wave owns a 128 x 128 block of the tile as 8 x 8 accumulators of
//    16 x 16 (256 registers).  A 64-deep slice is two K steps of 32; a K step
//    is 64 products, walked in four quadrants -- (A rows 0-3, B rows 0-3),
//    (A 0-3, B 4-7), (A 4-7, B 0-3), (A 4-7, B 4-7) in 16-row blocks -- each
//    A block by A block, so that consecutive products share the
//    instruction's second operand.
//  * One register set of 8 A and 8 B fragments (64 registers): each fragment
//    is read again for the next K step right after its last product of this
//    one.  In the quadrant order every such read has at least 20 products
//    (about 320 cycles) before its first use.
//  * Two ring stages of 64 KiB.  Stage g % 2 holds slice g; the hand-off of
//    slice g (this wave's copies of slice g + 1 landed, then a workgroup
//    barrier) sits after the 9th product of its second K step, before the
//    first read of slice g + 1 (after the 20th).  The 16 copies per wave of
//    slice g + 2 go out one after every fifth product from there on (11 in
//    this K step, 5 in the first K step of slice g + 1), so the address unit
//    sees a steady stream and the last copy has about 50 products to land.
//    (With the products B block by B block, a hand-off after product 28, 20
//    or 12 ran 0.2-1 % slower than after product 8.)
//  * The epilogue stages 32 (fp32: 16) rows of a wave's output at a time
//    through a wave-private LDS area and stores whole 256-byte row segments.
#pragma once

#include <type_traits>

#include "gemm_kernel.h"

namespace tcm {

struct Op16BF16 {
    static constexpr bool kScaled = false;
    static constexpr int kElemBits = 16;
    typedef bf16x8_t frag_t;
    __device__ static __forceinline__ f32x4_t mma(frag_t a, frag_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
struct Op16F16 {
    static constexpr bool kScaled = false;
    static constexpr int kElemBits = 16;
    typedef f16x8_t frag_t;
    __device__ static __forceinline__ f32x4_t mma(frag_t a, frag_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
// MXFP4 (E2M1 x E2M1, one E8M0 scale per 32) on v_mfma_scale_f32_16x16x128:
// lane l + 16 b holds the 32 K values of block b of row l % 16 in 16 bytes
// (the operand's first four registers) and supplies that block's scale, so a
// 128-deep K step of a 256-deep slice is laid out like a bf16 K step of 32.
struct Op16MXFP4 {
    static constexpr bool kScaled = true;
    static constexpr int kElemBits = 4;
    typedef i32x4_t frag_t;
    __device__ static __forceinline__ f32x4_t mma(frag_t a, frag_t b, f32x4_t c, int sa, int sb) {
        const i32x8_t a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
        const i32x8_t b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);
        // format codes 4 / 4: both operands FP4 E2M1
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
    }
};

// Schedule of one K step (slot x = after the x-th product, 0 .. 63).
namespace g16 {
constexpr int kHandoff = 8;                     // second K step: hand-off after product 8
constexpr int kCopyStep = 5;                    // one copy after every fifth product
constexpr int kCopyFirst1 = 10, kCopies1 = 11; // second K step: copies 0..10 of slice g + 2
constexpr int kCopyFirst0 = 1, kCopies0 = 5;   // first K step: copies 11..15 of slice g + 1
// product x: quadrant q = x / 16 (A half q / 2, B half q % 2), A block
// (x % 16) / 4 within the half, B block x % 4 within the half: four
// consecutive products share their A fragment, the instruction's second
// operand.  (With register operands only, products that keep the second
// operand for eight in a row sustain 2120 TFLOP/s, those that keep the first
// 1935: the matrix core's power, and so the clock, depends on which operand
// changes.)
__device__ constexpr int a_of(int x) { return 4 * ((x >> 4) >> 1) + ((x & 15) >> 2); }
__device__ constexpr int b_of(int x) { return 4 * ((x >> 4) & 1) + (x & 3); }
// fragment read for the next K step after product x (-1: none), right after
// the fragment's last product: A block i after product 19 + 4 i (i < 4) or
// 35 + 4 i; B block j after product 44 + j (j < 4) or 56 + j.  Each read has
// at least 20 products before its first use.
__device__ constexpr int a_read(int x) {
    return (x >= 19 && x <= 31 && (x - 19) % 4 == 0) ? (x - 19) / 4
           : (x >= 51 && (x - 51) % 4 == 0)          ? (x - 35) / 4
                                                     : -1;
}
__device__ constexpr int b_read(int x) { return (x >= 44 && x < 48) ? x - 44 : (x >= 60 ? x - 56 : -1); }
__device__ constexpr int copy1(int x) {
    return (x >= kCopyFirst1 && (x - kCopyFirst1) % kCopyStep == 0 &&
            (x - kCopyFirst1) / kCopyStep < kCopies1)
               ? (x - kCopyFirst1) / kCopyStep
               : -1;
}
__device__ constexpr int copy0(int x) {
    return (x >= kCopyFirst0 && (x - kCopyFirst0) % kCopyStep == 0 &&
            (x - kCopyFirst0) / kCopyStep < kCopies0)
               ? kCopies1 + (x - kCopyFirst0) / kCopyStep
               : -1;
}
constexpr int kLastCopy0 = kCopyFirst0 + (kCopies0 - 1) * kCopyStep;
constexpr int kScaleSlot = 12;  // second K step: MX scale chunk DMA (between two copies)
static_assert(kCopies1 + kCopies0 == 16, "16 copies per wave per slice");
static_assert(kCopyFirst1 > kHandoff && kCopyFirst1 + (kCopies1 - 1) * kCopyStep < 64, "copy slots");
static_assert(kLastCopy0 < 64, "copy slots");
}  // namespace g16

template <class Op, typename TOut>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm16_kernel(GemmArgs p) {
    constexpr bool SCALED = Op::kScaled;
    constexpr int EBITS = Op::kElemBits;
    constexpr int BM = 256, BN = 256, S = 2;
    constexpr int RB = 128;                // bytes of one row's slice
    constexpr int BK = RB * 8 / EBITS;     // K per slice: 64 (16-bit), 256 (FP4)
    constexpr int EPC = 128 / EBITS;       // elements per 16-byte chunk
    constexpr int A_BYTES = BM * RB;       // 32 KiB
    constexpr int STAGE = A_BYTES + BN * RB;
    constexpr int ROWS_PER_COPY = 8;       // a copy: 64 lanes x 16 bytes = 8 rows of 128 bytes
    // MX scales: 16-byte pieces of each A and B row (16 blocks of 32, SPC
    // slices) in two chunk buffers after the ring
    constexpr int CHUNK = (BM + BN) * 16;
    constexpr int SC_BYTES = SCALED ? 2 * CHUNK : 0;
    constexpr int SPC = 512 / BK;
    // output staging: 32 rows per wave, 16 beside the scale chunks (none for
    // fp32 there: direct stores)
    constexpr int STG_ROWS = SCALED ? (sizeof(TOut) == 2 ? 16 : 0) : (sizeof(TOut) == 2 ? 32 : 16);
    constexpr int STG_ROWB = 128 * (int)sizeof(TOut);
    constexpr int STG_BYTES = STG_ROWS * STG_ROWB;
    static_assert(S * STAGE + SC_BYTES + 4 * STG_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char lds[S * STAGE + SC_BYTES + 4 * STG_BYTES];
    char* const scb = lds + S * STAGE;  // scale chunk buffers (SCALED)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const int G = gridDim.x;
    const int lid = logical_block(blockIdx.x, G);
    if (lid >= p.total_tiles) return;
    const int my_tiles = (p.total_tiles - 1 - lid) / G + 1;
    const int total = my_tiles * p.ksteps;
    const int K = p.K;
    const uint32_t ROWB = (uint32_t)K * EBITS / 8;  // bytes of one operand row

    // ---- copies ----------------------------------------------------------
    // Copy x (0..15) of wave w fills LDS chunk q = (4 (x % 8) + w) * 64 + lane
    // of the A (x < 8) or B region: row q / 8, physical chunk q % 8, which
    // holds logical chunk (q % 8) ^ ((row / 2) % 8) of the row's slice.  The
    // logical chunk does not depend on x, and copy x + 1 sits 32 rows below x.
    const int cp_row = wave * ROWS_PER_COPY + lane / 8;
    const int cp_chunk = (lane & 7) ^ ((cp_row >> 1) & 7);
    const uint32_t cp_off = (uint32_t)cp_row * ROWB + (uint32_t)cp_chunk * 16u;
    const uint32_t cp_step = 32u * ROWB;

    TileCursor fc = {0, 0, 0, 0, 0};
    auto locate = [&](TileCursor& c) { tile_coords(p, c.tl * G + lid, c.batch, c.tm, c.tn); };
    __amdgpu_buffer_rsrc_t ra, rb;
    auto feed_resources = [&]() {
        const char* abase = (const char*)p.A + fc.batch * p.stride_a;
        const char* bbase = (const char*)p.B + fc.batch * p.stride_b;
        const int rows_a = min(BM, p.M - fc.tm * BM), rows_b = min(BN, p.N - fc.tn * BN);
        ra = make_rsrc(abase + (int64_t)fc.tm * BM * ROWB, (uint32_t)rows_a * ROWB);
        rb = make_rsrc(bbase + (int64_t)fc.tn * BN * ROWB, (uint32_t)rows_b * ROWB);
    };
    // buffer offset of copy 0 of the stream's slice; past the last slice, or
    // for a chunk past K, out of range (zeros, no memory touched)
    uint32_t foff0 = 0;
    auto feed_offsets = [&](bool live) {
        const bool kin = fc.kk * BK + cp_chunk * EPC < K;
        foff0 = live && kin ? cp_off + (uint32_t)(fc.kk * RB) : kOutOfRange;
    };
    int fg = 0;  // the copy stream's slice
    auto feed_next = [&]() {
        if (++fc.kk == p.ksteps) {
            fc.kk = 0;
            if (++fc.tl < my_tiles) {
                locate(fc);
                feed_resources();
            }
        }
        ++fg;
        feed_offsets(fg < total);
    };
    auto copy = [&](int st, int x) {
        char* dst = lds + st * STAGE + (x < 8 ? 0 : A_BYTES) + (4 * (x & 7) + wave) * 1024;
        copy16_to_lds(x < 8 ? ra : rb, dst, foff0 + (uint32_t)(x & 7) * cp_step);
    };

    // ---- MX scale chunks (SCALED) ---------------------------------------------
    // Chunk c of a tile: bytes 16 c .. 16 c + 15 of each scale row, the blocks
    // of slices SPC c .. SPC c + SPC - 1.  Copy q (0..7) of the workgroup
    // takes rows 64 q .. 64 q + 63 of the tile's A rows (q < 4) then B rows,
    // one row per lane; wave w issues copies w and w + 4.
    const int KS = K / 32;  // scale bytes per row
    TileCursor sc = {0, 0, 0, 0, 0};
    __amdgpu_buffer_rsrc_t rsa, rsb;
    auto scale_resources = [&]() {
        if constexpr (SCALED) {
            const int rows_a = min(BM, p.M - sc.tm * BM), rows_b = min(BN, p.N - sc.tn * BN);
            rsa = make_rsrc((const char*)p.SA + (int64_t)sc.tm * BM * KS, (uint32_t)rows_a * (uint32_t)KS);
            rsb = make_rsrc((const char*)p.SB + (int64_t)sc.tn * BN * KS, (uint32_t)rows_b * (uint32_t)KS);
        }
    };
    int sg = 0;  // the scale stream's first slice
    auto scale_copy = [&](int buf) {
        if constexpr (SCALED) {
            const bool live = sg < total;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q = wave + 4 * h;
                const uint32_t off = live ? (uint32_t)((q & 3) * 64 + lane) * (uint32_t)KS +
                                                (uint32_t)(sc.kk / SPC) * 16u
                                          : kOutOfRange;
                copy16_to_lds(q < 4 ? rsa : rsb, scb + buf * CHUNK + q * 1024, off);
            }
        }
    };
    auto scale_next = [&]() {
        sc.kk += SPC;
        sg += SPC;
        if (sc.kk == p.ksteps) {
            sc.kk = 0;
            if (++sc.tl < my_tiles) {
                locate(sc);
                scale_resources();
            }
        }
    };

    // ---- fragments ---------------------------------------------------------
    // 16 x 16 x 32 operands: lane l holds row l % 16 of a 16-row block, K
    // values 8 (l / 16) .. + 7 of the K step, i.e. logical chunk 4 s + l / 16
    // of the row's slice, stored at chunk ^ ((row / 2) % 8) = chunk ^ ((l % 16) / 2).
    const int r16 = lane & 15, g4 = lane >> 4;
    const int xr = r16 >> 1;
    const uint32_t a_row = (uint32_t)(wm * 128 + r16) * RB;
    const uint32_t b_row = (uint32_t)A_BYTES + (uint32_t)(wn * 128 + r16) * RB;
    const uint32_t ch0 = (uint32_t)((0 + g4) ^ xr) * 16u, ch1 = (uint32_t)((4 + g4) ^ xr) * 16u;
    // Accumulators: D = B_frag . A_frag^T per 16 x 16 block (operands
    // swapped), so lane l holds output row 16 i + l % 16 and the four
    // consecutive columns 16 j + 4 (l / 16) + 0..3.
    f32x4_t acc[8][8];
    typedef typename Op::frag_t frag_t;
    frag_t fa[8], fb[8];
    // MX: the scale byte of block 4 s + l / 16 of slice h for each fragment:
    // chunk buffer (h / SPC) % 2, byte 8 (h % SPC) + 4 s + l / 16 of the
    // row's piece (16 lanes read 16 rows 16 bytes apart: 16 different banks)
    int sa[8], sb[8];
    const uint32_t sa_row = (uint32_t)(wm * 128 + r16) * 16u + (uint32_t)g4;
    const uint32_t sb_row = 4096u + (uint32_t)(wn * 128 + r16) * 16u + (uint32_t)g4;
    auto scale_at = [&](int h, int s) -> const char* {
        return scb + ((h / SPC) & 1) * CHUNK + 8 * (h % SPC) + 4 * s;
    };
    // fragment i (j) of K step s of slice h, from stage h % 2
    auto read_a = [&](int h, int s, int i) {
        fa[i] = *(const frag_t*)(lds + (h & 1) * STAGE + a_row + i * 16 * RB + (s ? ch1 : ch0));
        if constexpr (SCALED) sa[i] = *(const unsigned char*)(scale_at(h, s) + sa_row + i * 256);
    };
    auto read_b = [&](int h, int s, int j) {
        fb[j] = *(const frag_t*)(lds + (h & 1) * STAGE + b_row + j * 16 * RB + (s ? ch1 : ch0));
        if constexpr (SCALED) sb[j] = *(const unsigned char*)(scale_at(h, s) + sb_row + j * 256);
    };
    auto mma = [&](int i, int j, f32x4_t c) {
        if constexpr (SCALED)
            acc[i][j] = Op::mma(fb[j], fa[i], c, sb[j], sa[i]);
        else
            acc[i][j] = Op::mma(fb[j], fa[i], c);
    };


    // ---- epilogue ----------------------------------------------------------
    auto epilogue = [&](const TileCursor& c) {
        const int ldc = p.N;
        char* Cb = (char*)p.C + c.batch * p.stride_c;
        const int m0 = c.tm * BM + wm * 128, n0 = c.tn * BN + wn * 128;
        const bool full = c.tm * BM + BM <= p.M && c.tn * BN + BN <= p.N;
        if (STG_ROWS > 0 && full && ldc % (16 / (int)sizeof(TOut)) == 0) {
            constexpr int CHK = STG_ROWB / 16;              // 16-byte chunks per staged row
            constexpr int RPI = kWaveSize * 16 / STG_ROWB;  // rows per read-back instruction
            constexpr int IPP = STG_ROWS > 0 ? STG_ROWS / 16 : 1;  // 16-row blocks per pass
            char* stg = lds + S * STAGE + SC_BYTES + wave * STG_BYTES;
            // the lane index afresh (offsets kept from the kernel's start
            // would hold registers across the K loop)
            const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
            const int rr = ln & 15, gg = ln >> 4;
#pragma unroll
            for (int ps = 0; ps < (STG_ROWS > 0 ? 8 / IPP : 0); ++ps) {
#pragma unroll
                for (int ii = 0; ii < IPP; ++ii)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const f32x4_t v = acc[IPP * ps + ii][j];
                        const int row = 16 * ii + rr;
                        const int byte = (16 * j + 4 * gg) * (int)sizeof(TOut);
                        const int chunk = (byte / 16) ^ (row & 15);
                        store4<TOut>((TOut*)(stg + row * STG_ROWB + chunk * 16 + byte % 16), v[0], v[1],
                                     v[2], v[3]);
                    }
                wave_lds_exchange();
#pragma unroll
                for (int t = 0; t < STG_ROWS / RPI; ++t) {
                    const int r = t * RPI + ln / CHK;
                    const int ck = ln % CHK;
                    const i32x4_t d = *(const i32x4_t*)(stg + r * STG_ROWB + ((ck ^ (r & 15)) * 16));
                    char* gp = Cb + ((int64_t)(m0 + STG_ROWS * ps + r) * ldc + n0) * (int64_t)sizeof(TOut) +
                               ck * 16;
                    // non-temporal: the output does not displace operand rows in L2
                    __builtin_nontemporal_store(d, (i32x4_t*)gp);
                }
                wave_lds_exchange();
            }
            return;
        }
        // edge tile (or rows not 16-byte aligned): rows past M and columns
        // past N are not written
        const bool vec = (ldc & 3) == 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int m = m0 + 16 * i + r16;
            if (m >= p.M) continue;
            TOut* row = (TOut*)Cb + (int64_t)m * ldc;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int n = n0 + 16 * j + 4 * g4;
                const f32x4_t v = acc[i][j];
                if (vec && n + 3 < p.N) {
                    store4<TOut>(row + n, v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) row[n + e] = convert_out<TOut>(v[e]);
                }
            }
        }
    };

    // ---- the K steps ---------------------------------------------------------
    // First K step of slice g: reads of K step 1 (stage g % 2), copies 11..15
    // of slice g + 1 (stage (g + 1) % 2), then the stream moves to slice g + 2.
    auto step0 = [&](int g, auto ZERO) {
        const int st = g & 1;
        static_for<64>([&](auto X) {
            constexpr int x = decltype(X)::value;
            constexpr int i = g16::a_of(x), j = g16::b_of(x);
            mma(i, j, decltype(ZERO)::value ? (f32x4_t){} : acc[i][j]);
            if constexpr (g16::copy0(x) >= 0) copy(st ^ 1, g16::copy0(x));
            if constexpr (x == g16::kLastCopy0) feed_next();
            if constexpr (g16::a_read(x) >= 0) read_a(g, 1, g16::a_read(x));
            if constexpr (g16::b_read(x) >= 0) read_b(g, 1, g16::b_read(x));
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // Second K step of slice g: hand-off, then copies 0..10 of slice g + 2
    // (stage g % 2) and reads of slice g + 1's first K step (stage (g + 1) % 2).
    auto step1 = [&](int g) {
        const int st = g & 1;
        static_for<64>([&](auto X) {
            constexpr int x = decltype(X)::value;
            constexpr int i = g16::a_of(x), j = g16::b_of(x);
            mma(i, j, acc[i][j]);
            if constexpr (x == g16::kHandoff) {
                wait_vmcnt<0>();
                barrier_lds();
            }
            if constexpr (g16::copy1(x) >= 0) copy(st, g16::copy1(x));
            if constexpr (SCALED && x == g16::kScaleSlot) {
                // the chunk buffer of slices g + SPC .. held slices g - SPC ..,
                // whose last scale reads preceded this hand-off
                if (g % SPC == 0) {
                    scale_copy((g / SPC + 1) & 1);
                    scale_next();
                }
            }
            if constexpr (g16::a_read(x) >= 0) read_a(g + 1, 0, g16::a_read(x));
            if constexpr (g16::b_read(x) >= 0) read_b(g + 1, 0, g16::b_read(x));
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ---- prologue: slice 0 whole, copies 0..10 of slice 1 --------------------
    locate(fc);
    feed_resources();
    feed_offsets(true);
    sc = fc;
    scale_resources();
#pragma unroll
    for (int x = 0; x < 16; ++x) copy(0, x);
    if constexpr (SCALED) {
        scale_copy(0);
        scale_next();
    }
    feed_next();
#pragma unroll
    for (int x = 0; x < g16::kCopies1; ++x) copy(1, x);
    wait_vmcnt<g16::kCopies1>();  // (slice 0 and the first scale chunk)
    barrier_lds();
#pragma unroll
    for (int i = 0; i < 8; ++i) read_a(0, 0, i);
#pragma unroll
    for (int j = 0; j < 8; ++j) read_b(0, 0, j);

    int g = 0;
    for (int tl = 0; tl < my_tiles; ++tl) {
        step0(g, std::true_type{});
        step1(g);
        ++g;
        for (int kk = 1; kk < p.ksteps; ++kk, ++g) {
            step0(g, std::false_type{});
            step1(g);
        }
        TileCursor ec = {tl, 0, 0, 0, 0};
        locate(ec);
        __builtin_amdgcn_sched_barrier(0);
        epilogue(ec);
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace tcm
