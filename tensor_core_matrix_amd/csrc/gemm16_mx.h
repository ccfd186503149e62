// The 256 x 256 MXFP8 product (E4M3 x E4M3, one E8M0 scale per 32 K values)
// on the 16 x 16 x 128 scaled matrix-core instruction of gfx950
// (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// "Hopper and Blackwell GEMM" ("FP8 and FP4, with block scaling") applies the
// block scales inside the tensor-core instruction.  A 128-deep fp8 slice has
// the bytes of a 64-deep bf16 slice, so this kernel is the one of gemm16.h
// with one K step per slice: 8 x 8 products of 16 x 16 x 128 per wave, 32
// cycles each (the same 2048 cycles per slice), the same LDS rows, swizzle,
// copy stream and quadrant order, and fragments refilled after their last
// product.  Per slice and wave:
//
//  * the hand-off (this wave's copies of slice g + 1 landed, workgroup
//    barrier) after product 8, then the 16 copies of slice g + 2 into the
//    freed stage, one after every third product;
//  * a fragment is 32 bytes per lane (lane l: row l % 16 of its 16-row block,
//    16-byte K chunks l / 16 and 4 + l / 16 of the slice, two ds_read_b128),
//    and lane l + 16 b supplies the scale of K block b of row l % 16;
//  * scales travel by DMA: every fourth slice one 16-byte piece per A and B
//    row (the scale blocks of four slices) goes to one of two 8 KiB chunk
//    buffers, and each lane reads the byte of its row and block for the next
//    slice with a ds_read_u8 (16 lanes read 16 rows 16 bytes apart: 16
//    different banks).
//
// Requires K % 512 == 0 and 16-byte aligned scale arrays (whole 16-byte
// pieces per row); dense storage (rows K apart, Out rows N apart).
//
// MXFP6 (FMT 2: E2M3, 3: E3M2) runs the same kernel.  Lane l + 16 b of a
// 16 x 16 x 128 product holds the whole block b of its row: 32 six-bit codes
// as the block's 24 stored bytes in the operand's first six registers (as in
// the 32 x 32 x 64 form, one lane group per block).  A 128-deep slice is 96
// bytes of a stored row.  Its LDS row keeps the 128 bytes and 8 chunks of the
// fp8 layout: chunk b < 4 holds bytes 0-15 of block b, chunk 4 + b the 16
// stored bytes from byte 8 of block b (b = 0, 3: the block's last 8 bytes in
// the chunk's upper half) or from byte 16 (b = 1, 2: in its lower half,
// followed by the next block's first 8).  A fragment is a 16-byte read of
// chunk b and an 8-byte read of the block's last 8 bytes from chunk 4 + b;
// the 32 lanes served together by an 8-byte read (blocks 0 and 1, or 2 and
// 3) use opposite halves of their chunks and so meet no bank twice.  Every
// copy stays inside its row's slice.  A product takes half the cycles of an
// fp8 one, so the same copy stream serves twice the products per cycle.
#pragma once

#include "gemm16.h"

namespace tcm {

namespace g16mx {
constexpr int kHandoff = 8;
constexpr int kCopyFirst = 10, kCopyStep = 3;  // copies 0..15 of slice g + 2 after products 10, 13, .., 55
constexpr int kLastCopy = kCopyFirst + 15 * kCopyStep;
constexpr int kScaleSlot0 = 57, kScaleSlot1 = 59;  // scale chunk DMA (first slice of a chunk)
__device__ constexpr int copy_at(int x) {
    return (x >= kCopyFirst && (x - kCopyFirst) % kCopyStep == 0 && (x - kCopyFirst) / kCopyStep < 16)
               ? (x - kCopyFirst) / kCopyStep
               : -1;
}
static_assert(kLastCopy < 64 && kScaleSlot1 < 64, "slots");
// MXFP6: the stored byte of a slice row that LDS chunk c (0..7) starts at
__device__ constexpr int f6_chunk(int c) {
    return c < 4 ? 24 * c : 24 * (c - 4) + ((c == 4 || c == 7) ? 8 : 16);
}
static_assert(f6_chunk(7) + 16 == 96 && f6_chunk(6) + 16 <= 96, "MXFP6 chunks stay inside the slice");
}  // namespace g16mx

// FMT: the operands' format code of the scaled product, 0 E4M3, 2 E2M3, 3 E3M2
template <typename TOut, int FMT = 0>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm16_mx_kernel(GemmArgs p) {
    static_assert(FMT == 0 || FMT == 2 || FMT == 3, "E4M3, E2M3 or E3M2");
    constexpr bool F6 = FMT != 0;
    constexpr int BM = 256, BN = 256, BK = 128, S = 2;
    constexpr int RB = BK;                 // LDS bytes of one row's slice
    constexpr int RBG = F6 ? 96 : 128;     // stored bytes of one row's slice
    constexpr int A_BYTES = BM * RB;       // 32 KiB
    constexpr int STAGE = A_BYTES + BN * RB;
    constexpr int CHUNK = (BM + BN) * 16;  // scale bytes of four slices, 8 KiB
    constexpr bool EPI_LDS = sizeof(TOut) == 2;
    constexpr int STG_ROWB = 128 * (int)sizeof(TOut);
    constexpr int STG_BYTES = EPI_LDS ? 16 * STG_ROWB : 0;  // 16 rows per wave
    static_assert(S * STAGE + 2 * CHUNK + 4 * STG_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char lds[S * STAGE + 2 * CHUNK + 4 * STG_BYTES];
    char* const scb = lds + S * STAGE;  // the two chunk buffers

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
    const int KS = K / 32;  // scale bytes per row
    const int RS = F6 ? K / 4 * 3 : K;  // stored bytes per row

    // ---- operand copies (as gemm16.h, 128 values per row and slice) --------
    const int cp_row = wave * 8 + lane / 8;
    const int cp_chunk = (lane & 7) ^ ((cp_row >> 1) & 7);
    const uint32_t cp_byte = F6 ? (uint32_t)g16mx::f6_chunk(cp_chunk) : (uint32_t)cp_chunk * 16u;
    const uint32_t cp_off = (uint32_t)cp_row * (uint32_t)RS + cp_byte;
    const uint32_t cp_step = 32u * (uint32_t)RS;

    auto locate = [&](TileCursor& c) { tile_coords(p, c.tl * G + lid, c.batch, c.tm, c.tn); };
    TileCursor fc = {0, 0, 0, 0, 0};
    __amdgpu_buffer_rsrc_t ra, rb;
    auto feed_resources = [&]() {
        const int rows_a = min(BM, p.M - fc.tm * BM), rows_b = min(BN, p.N - fc.tn * BN);
        ra = make_rsrc((const char*)p.A + (int64_t)fc.tm * BM * RS, (uint32_t)rows_a * (uint32_t)RS);
        rb = make_rsrc((const char*)p.B + (int64_t)fc.tn * BN * RS, (uint32_t)rows_b * (uint32_t)RS);
    };
    uint32_t foff0 = 0;
    int fg = 0;
    auto feed_offsets = [&]() { foff0 = fg < total ? cp_off + (uint32_t)(fc.kk * RBG) : kOutOfRange; };
    auto feed_next = [&]() {
        if (++fc.kk == p.ksteps) {
            fc.kk = 0;
            if (++fc.tl < my_tiles) {
                locate(fc);
                feed_resources();
            }
        }
        ++fg;
        feed_offsets();
    };
    auto copy = [&](int st, int x) {
        char* dst = lds + st * STAGE + (x < 8 ? 0 : A_BYTES) + (4 * (x & 7) + wave) * 1024;
        copy16_to_lds(x < 8 ? ra : rb, dst, foff0 + (uint32_t)(x & 7) * cp_step);
    };

    // ---- scale chunks ------------------------------------------------------
    // Chunk c of a tile: bytes 16 c .. 16 c + 15 of each scale row, the
    // blocks of slices 4 c .. 4 c + 3.  Copy q (0..7) of the workgroup takes
    // rows 64 q .. 64 q + 63 of the tile's A rows (q < 4) then B rows, one row
    // per lane; wave w issues copies w and w + 4.  The scale stream `sc` runs
    // four slices ahead of the slice it is issued in.
    TileCursor sc = {0, 0, 0, 0, 0};
    __amdgpu_buffer_rsrc_t rsa, rsb;
    auto scale_resources = [&]() {
        const int rows_a = min(BM, p.M - sc.tm * BM), rows_b = min(BN, p.N - sc.tn * BN);
        rsa = make_rsrc((const char*)p.SA + (int64_t)sc.tm * BM * KS, (uint32_t)rows_a * (uint32_t)KS);
        rsb = make_rsrc((const char*)p.SB + (int64_t)sc.tn * BN * KS, (uint32_t)rows_b * (uint32_t)KS);
    };
    int sg = 0;  // the scale stream's first slice
    auto scale_copy = [&](int buf) {
        const bool live = sg < total;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = wave + 4 * h;
            const uint32_t off = live ? (uint32_t)((q & 3) * 64 + lane) * (uint32_t)KS + (uint32_t)(sc.kk / 4) * 16u
                                      : kOutOfRange;
            copy16_to_lds(q < 4 ? rsa : rsb, scb + buf * CHUNK + q * 1024, off);
        }
    };
    auto scale_next = [&]() {
        sc.kk += 4;
        sg += 4;
        if (sc.kk == p.ksteps) {
            sc.kk = 0;
            if (++sc.tl < my_tiles) {
                locate(sc);
                scale_resources();
            }
        }
    };

    // ---- fragments and scale bytes -------------------------------------------
    const int r16 = lane & 15, g4 = lane >> 4;
    const int xr = r16 >> 1;
    const uint32_t a_row = (uint32_t)(wm * 128 + r16) * RB;
    const uint32_t b_row = (uint32_t)A_BYTES + (uint32_t)(wn * 128 + r16) * RB;
    const uint32_t ch0 = (uint32_t)(g4 ^ xr) * 16u;
    // MXFP6: the block's last 8 bytes sit at byte 8 of chunk 4 + b for b = 0, 3
    const uint32_t ch1 = (uint32_t)((4 + g4) ^ xr) * 16u + (F6 && (g4 == 0 || g4 == 3) ? 8u : 0u);
    const uint32_t sa_row = (uint32_t)(wm * 128 + r16) * 16u + (uint32_t)g4;
    const uint32_t sb_row = 4096u + (uint32_t)(wn * 128 + r16) * 16u + (uint32_t)g4;
    // the two 16-byte halves of each fragment are kept apart and joined at
    // the product (an 8-register value refilled in the loop made the compiler
    // move every fragment register at the loop's back edge)
    typedef typename std::conditional<F6, i32x2_t, i32x4_t>::type half_t;
    i32x4_t fa0[8], fb0[8];
    half_t fa1[8], fb1[8];
    int sa[8], sb[8];
    // fragments of slice h: stage h % 2; scales: chunk buffer (h / 4) % 2, byte 4 (h % 4) + l / 16
    auto read_a = [&](int h, int i) {
        const char* p0 = lds + (h & 1) * STAGE + a_row + i * 16 * RB;
        fa0[i] = *(const i32x4_t*)(p0 + ch0);
        fa1[i] = *(const half_t*)(p0 + ch1);
        sa[i] = *(const unsigned char*)(scb + ((h >> 2) & 1) * CHUNK + sa_row + i * 256 + 4 * (h & 3));
    };
    auto read_b = [&](int h, int j) {
        const char* p0 = lds + (h & 1) * STAGE + b_row + j * 16 * RB;
        fb0[j] = *(const i32x4_t*)(p0 + ch0);
        fb1[j] = *(const half_t*)(p0 + ch1);
        sb[j] = *(const unsigned char*)(scb + ((h >> 2) & 1) * CHUNK + sb_row + j * 256 + 4 * (h & 3));
    };

    // lane l: output row 16 i + l % 16, columns 16 j + 4 (l / 16) + 0..3
    f32x4_t acc[8][8];

    // ---- epilogue ------------------------------------------------------------
    auto epilogue = [&](const TileCursor& c) {
        const int ldc = p.N;
        char* Cb = (char*)p.C;
        const int m0 = c.tm * BM + wm * 128, n0 = c.tn * BN + wn * 128;
        const bool full = c.tm * BM + BM <= p.M && c.tn * BN + BN <= p.N;
        if constexpr (EPI_LDS) {
            if (full && ldc % 8 == 0) {
                constexpr int CHK = STG_ROWB / 16;              // 16 chunks per staged row
                constexpr int RPI = kWaveSize * 16 / STG_ROWB;  // 4 rows per read-back
                char* stg = lds + S * STAGE + 2 * CHUNK + wave * STG_BYTES;
                const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
                const int rr = ln & 15, gg = ln >> 4;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const f32x4_t v = acc[i][j];
                        const int byte = (16 * j + 4 * gg) * (int)sizeof(TOut);
                        const int chunk = (byte / 16) ^ rr;
                        store4<TOut>((TOut*)(stg + rr * STG_ROWB + chunk * 16 + byte % 16), v[0], v[1], v[2],
                                     v[3]);
                    }
                    wave_lds_exchange();
#pragma unroll
                    for (int t = 0; t < 16 / RPI; ++t) {
                        const int r = t * RPI + ln / CHK;
                        const int ck = ln % CHK;
                        const i32x4_t d = *(const i32x4_t*)(stg + r * STG_ROWB + ((ck ^ r) * 16));
                        char* gp = Cb + ((int64_t)(m0 + 16 * i + r) * ldc + n0) * (int64_t)sizeof(TOut) + ck * 16;
                        // non-temporal: the output does not displace operand rows in L2
                        __builtin_nontemporal_store(d, (i32x4_t*)gp);
                    }
                    wave_lds_exchange();
                }
                return;
            }
        }
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

    // ---- one slice -------------------------------------------------------------
    auto slice = [&](int g, auto ZERO) {
        const int st = g & 1;
        const bool chunk_slice = (g & 3) == 0;
        static_for<64>([&](auto X) {
            constexpr int x = decltype(X)::value;
            constexpr int i = g16::a_of(x), j = g16::b_of(x);
            const f32x4_t c = decltype(ZERO)::value ? (f32x4_t){} : acc[i][j];
            i32x8_t a8, b8;
            if constexpr (F6) {
                // registers 0-5: the block's 24 bytes; 6, 7 unused
                a8 = __builtin_shufflevector(fa0[i], __builtin_shufflevector(fa1[i], fa1[i], 0, 1, -1, -1), 0, 1,
                                             2, 3, 4, 5, -1, -1);
                b8 = __builtin_shufflevector(fb0[j], __builtin_shufflevector(fb1[j], fb1[j], 0, 1, -1, -1), 0, 1,
                                             2, 3, 4, 5, -1, -1);
            } else {
                a8 = __builtin_shufflevector(fa0[i], fa1[i], 0, 1, 2, 3, 4, 5, 6, 7);
                b8 = __builtin_shufflevector(fb0[j], fb1[j], 0, 1, 2, 3, 4, 5, 6, 7);
            }
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, c, FMT, FMT, 0, sb[j], 0, sa[i]);
            if constexpr (x == g16mx::kHandoff) {
                wait_vmcnt<0>();
                barrier_lds();
            }
            if constexpr (g16mx::copy_at(x) >= 0) copy(st, g16mx::copy_at(x));
            if constexpr (x == g16mx::kLastCopy) feed_next();
            if constexpr (x == g16mx::kScaleSlot0) {
                // the chunk buffer of slices g + 4 .. g + 7 held slices g - 4 .. g - 1,
                // whose last reads preceded this slice's hand-off
                if (chunk_slice) {
                    scale_copy(((g >> 2) + 1) & 1);
                    scale_next();
                }
            }
            if constexpr (g16::a_read(x) >= 0) read_a(g + 1, g16::a_read(x));
            if constexpr (g16::b_read(x) >= 0) read_b(g + 1, g16::b_read(x));
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ---- prologue: slice 0 and scale chunk 0, then slice 1 --------------------
    locate(fc);
    feed_resources();
    feed_offsets();
    sc = fc;
    scale_resources();
#pragma unroll
    for (int x = 0; x < 16; ++x) copy(0, x);
    scale_copy(0);
    scale_next();
    feed_next();
#pragma unroll
    for (int x = 0; x < 16; ++x) copy(1, x);
    feed_next();
    wait_vmcnt<16>();
    barrier_lds();
#pragma unroll
    for (int i = 0; i < 8; ++i) read_a(0, i);
#pragma unroll
    for (int j = 0; j < 8; ++j) read_b(0, j);

    int g = 0;
    for (int tl = 0; tl < my_tiles; ++tl) {
        slice(g, std::true_type{});
        ++g;
        if constexpr (F6) {
            // two slices per iteration: with one, the compiler moved ten
            // fragments' registers at every back edge (MXFP8's 8-register
            // fragments do not fit two slices' worth and spill)
            int kk = 1;
            for (; kk + 1 < p.ksteps; kk += 2, g += 2) {
                slice(g, std::false_type{});
                slice(g + 1, std::false_type{});
            }
            if (kk < p.ksteps) {
                slice(g, std::false_type{});
                ++g;
            }
        } else {
            for (int kk = 1; kk < p.ksteps; ++kk, ++g) slice(g, std::false_type{});
        }
        TileCursor ec = {tl, 0, 0, 0, 0};
        locate(ec);
        __builtin_amdgcn_sched_barrier(0);
        epilogue(ec);
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace tcm
