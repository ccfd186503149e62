// NVFP4 (E2M1 elements, an E4M3 scale per 16, an fp32 scale per tensor) on
// the 16 x 16 x 32 fp16 matrix-core instruction, with the elements kept in
// their 4-bit form all the way to the registers.
//
// No matrix-core form takes E4M3 block scales ("Hopper and Blackwell GEMM",
// Concept, "FP8 and FP4, with block scaling": the format table's NVFP4 row),
// but an E2M1 value times an E4M3 scale is exact in fp16.  The register-staged
// kernel of gemm_kernel.h dequantizes while copying, so its LDS tiles and its
// copy stream carry fp16: four times the bytes of the data.  Here the copies
// move the 4-bit rows by DMA, as for MXFP4 (gemm16.h), and each lane converts
// its own fragments just before the products that use them:
//
//  * Slices are 256 deep (128-byte rows, two 64 KiB ring stages, the swizzle
//    and tile order of gemm16.h); a slice is eight K steps of 32, each 64
//    products of 16 x 16 x 32 walked in gemm16.h's quadrant order.  The loop
//    body is a pair of K steps (a body of four pairs, 512 products, defeats
//    the register allocator: it moves accumulators at every back edge).
//  * Lane l + 16 g of a fragment takes, for K steps 2 n and 2 n + 1 of a
//    slice, 8 bytes of row l: half h = (n + g) % 2 of 16-byte chunk
//    4 (n / 2) + g, i.e. the 16 E2M1 values of block 8 (n / 2) + 2 g + h,
//    values 0-7 for the first K step and 8-15 for the second, and that
//    block's scale byte.  (With h = n % 2 for every lane, the 32 lanes that
//    an 8-byte LDS read serves at once would meet each bank twice.)  The
//    matrix core sums a K step over its 32 positions whatever K values they
//    hold, so a K step sums its own 32 K values of the slice and the eight K
//    steps all 256: the same sum in another order.
//  * A fragment of a K step is four v_cvt_scalef32_pk_f16_fp4 (two values
//    each; the instruction's scale operand applies only a power of two, so
//    it is 1) and four fp16 multiplications by the block scale (exact).  The
//    conversions for the next K step are spread one per product, each after
//    the fragment's last product of this K step, its multiplication one
//    product later.  A wave issues at most one instruction per 4 cycles, a
//    product takes 16: conversions, reads, copies and their address
//    arithmetic together must stay under three instructions per product.
//  * The hand-off of slice g (this wave's copies of slice g + 1 landed, then
//    the workgroup barrier) opens K step 6, after the last read of slice g's
//    stage and before the first read of slice g + 1.  Each pair then issues
//    four of the 16 element copies per wave of the slice two ahead, early in
//    its first K step, and the first two pairs one scale copy each.
//  * Block scales come by DMA as the row's 16 scale bytes of the slice (one
//    8 KiB piece buffer per stage); the epilogue multiplies by the product of
//    the tensor scales and stages 16 rows of 16-bit output per wave through
//    LDS (fp32 output is stored directly).
// One problem per launch (the NVFP4 entry point takes no batch); K a multiple
// of 256 and both scale tensors 16-byte aligned, as the host checks.
#pragma once

#include "gemm16.h"

namespace tcm {

namespace g16nv {
// Copies of slice g + 2, pair by pair: group q = (n + 1) % 4 of pair n
// (pair 3 of slice g, then pairs 0-2 of slice g + 1) is element copies
// 4 q .. 4 q + 3, after products 4, 20, 36 and 52 of the pair's first K step,
// and in groups 0 and 1 the scale copy q after product 4 of the second.
__device__ constexpr int copy_at(int x) { return x == 4 ? 0 : x == 20 ? 1 : x == 36 ? 2 : x == 52 ? 3 : -1; }
constexpr int kScaleCopySlot = 4;
// Conversion slots of fragment f (A blocks 0-7, then B blocks 8-15), part p
// (values 2p, 2p + 1 of the lane's 8): the product after which the part is
// converted, counted from the first product of K step t (for K step t + 1);
// 64 and up is the next K step itself.  Its scale multiplication follows
// after the next product.  A block i's last product in a K step is 19 + 4i
// (i < 4) or 35 + 4i and its first 4i or 16 + 4i; B block j's last 44 + j
// (j < 4) or 56 + j and its first j or 12 + j.  A part's slot lies after
// the fragment's last product and at least two before its first.
__device__ constexpr int conv_slot(int f, int p) {
    return f < 4    ? 20 + 4 * f + p                  // A0-A3: 20 .. 35
           : f < 6  ? 77 + 4 * (f - 4) + p - (f - 4)  // A4: 77-80, A5: 80-83
           : f < 8  ? 99 + 4 * (f - 6) + p            // A6, A7: 99 .. 106
           : f < 12 ? 45 + (f - 8) + 4 * p            // B0-B3: 45 .. 60
                    : 61 + (f - 12) + 4 * p;          // B4-B7: 61 .. 76
}
// the first product using fragment f in the K step after the one its
// conversion slots count from
__device__ constexpr int first_use(int f) {
    return 64 + (f < 4 ? 4 * f : f < 8 ? 16 + 4 * f : f < 12 ? f - 8 : 12 + (f - 8));
}
// A VALU result read by a product needs two wait states: s_nop operand after
// the multiplication of part p of fragment f (-1: none).  The multiplication
// runs after product conv_slot + 1.
__device__ constexpr int conv_nops(int f, int p) {
    return first_use(f) - conv_slot(f, p) == 2 ? 1 : -1;
}
// the last product using fragment f in the K step its slots count from
__device__ constexpr int last_use(int f) {
    return f < 4 ? 19 + 4 * f : f < 8 ? 35 + 4 * f : f < 12 ? 44 + (f - 8) : 56 + (f - 8);
}
// Every part after the fragment's last product and two before its first, the
// parts of a fragment in order, at most two conversions after one product.
__device__ constexpr bool slots_valid() {
    int per_slot[128] = {};
    for (int f = 0; f < 16; ++f)
        for (int p = 0; p < 4; ++p) {
            const int s = conv_slot(f, p);
            if (s <= last_use(f) || s + 2 > first_use(f) || s >= 128) return false;
            if (p > 0 && s < conv_slot(f, p - 1)) return false;
            if (++per_slot[s] > 2) return false;
        }
    for (int x = 0; x < 64; ++x)
        if (per_slot[x] + per_slot[x + 64] > 2) return false;
    return true;
}
static_assert(slots_valid(), "conversion slots");
static_assert(conv_slot(6, 3) + 2 == first_use(6) && conv_slot(7, 3) + 2 == first_use(7), "A6, A7 windows");
// the k-th conversion (4 f + p) at slot s, k = 0, 1 (at most two share a slot), or -1
__device__ constexpr int task_at(int s, int k) {
    int n = 0;
    for (int f = 0; f < 16; ++f)
        for (int p = 0; p < 4; ++p)
            if (conv_slot(f, p) == s) {
                if (n == k) return 4 * f + p;
                ++n;
            }
    return -1;
}
}  // namespace g16nv

// Byte P of w (two E2M1 values, the low nibble first) as two fp16 values;
// CVT: s holds an E4M3 byte (zero-extended) and is also made that fp16, in
// the low half.
template <int P, bool CVT>
__device__ __forceinline__ int fp4_pair(uint32_t w, int& s) {
    int r;
#define TCM_FP4_CVT(SEL)                                                                           \
    if constexpr (CVT)                                                                             \
        asm volatile("v_cvt_f32_fp8_e32 %1, %1\n\tv_cvt_scalef32_pk_f16_fp4 %0, %2, 1.0" SEL        \
                     "\n\tv_cvt_f16_f32_e32 %1, %1"                                                 \
                     : "=&v"(r), "+v"(s)                                                            \
                     : "v"(w));                                                                     \
    else                                                                                           \
        asm volatile("v_cvt_scalef32_pk_f16_fp4 %0, %1, 1.0" SEL : "=v"(r) : "v"(w))
    if constexpr (P == 0) {
        TCM_FP4_CVT("");
    } else if constexpr (P == 1) {
        TCM_FP4_CVT(" op_sel:[1,0,0]");
    } else if constexpr (P == 2) {
        TCM_FP4_CVT(" op_sel:[0,1,0]");
    } else {
        TCM_FP4_CVT(" op_sel:[1,1,0]");
    }
#undef TCM_FP4_CVT
    return r;
}

// v times the fp16 in the low half of s (both halves); NOP >= 0 appends
// s_nop NOP.
template <int NOP>
__device__ __forceinline__ int fp16x2_scaled(int v, int s) {
    int r;
    if constexpr (NOP >= 0)
        asm volatile("v_pk_mul_f16 %0, %1, %2 op_sel_hi:[0,1]\n\ts_nop %3"
                     : "=v"(r)
                     : "v"(s), "v"(v), "n"(NOP));
    else
        asm volatile("v_pk_mul_f16 %0, %1, %2 op_sel_hi:[0,1]" : "=v"(r) : "v"(s), "v"(v));
    return r;
}

template <typename TOut>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm16_nv4_kernel(GemmArgs p) {
    constexpr int BM = 256, BN = 256, S = 2;
    constexpr int RB = 128;              // bytes of one row's slice (256 E2M1 values)
    constexpr int A_BYTES = BM * RB;     // 32 KiB
    constexpr int STAGE = A_BYTES + BN * RB;
    constexpr int ROWS_PER_COPY = 8;
    constexpr int CHUNK = (BM + BN) * 16;  // a slice's scale pieces: 16 bytes per row
    constexpr int SC_BYTES = S * CHUNK;
    constexpr int STG_ROWS = sizeof(TOut) == 2 ? 16 : 0;
    constexpr int STG_ROWB = 128 * (int)sizeof(TOut);
    constexpr int STG_BYTES = STG_ROWS * STG_ROWB;
    static_assert(S * STAGE + SC_BYTES + 4 * STG_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char lds[S * STAGE + SC_BYTES + 4 * STG_BYTES];
    char* const scb = lds + S * STAGE;

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
    const uint32_t ROWB = (uint32_t)K / 2;    // bytes of one element row
    const uint32_t KS = (uint32_t)K / 16;     // bytes of one scale row (K a multiple of 256)

    // ---- copies (as gemm16.h): copy x (0..15) of wave w fills 1 KiB block
    // 4 (x % 8) + w of the A (x < 8) or B region, rows 8 (4 (x % 8) + w) .. + 7,
    // physical chunk l % 8 of each holding logical chunk (l % 8) ^ ((row / 2) % 8)
    const int cp_row = wave * ROWS_PER_COPY + lane / 8;
    const int cp_chunk = (lane & 7) ^ ((cp_row >> 1) & 7);
    const uint32_t cp_off = (uint32_t)cp_row * ROWB + (uint32_t)cp_chunk * 16u;
    const uint32_t cp_step = 32u * ROWB;

    TileCursor fc = {0, 0, 0, 0, 0};
    auto locate = [&](TileCursor& c) __attribute__((always_inline)) {
        tile_coords(p, c.tl * G + lid, c.batch, c.tm, c.tn);
    };
    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
    auto feed_resources = [&]() __attribute__((always_inline)) {
        const int rows_a = min(BM, p.M - fc.tm * BM), rows_b = min(BN, p.N - fc.tn * BN);
        ra = make_rsrc((const char*)p.A + (int64_t)fc.tm * BM * ROWB, (uint32_t)rows_a * ROWB);
        rb = make_rsrc((const char*)p.B + (int64_t)fc.tn * BN * ROWB, (uint32_t)rows_b * ROWB);
        rsa = make_rsrc((const char*)p.SA + (int64_t)fc.tm * BM * KS, (uint32_t)rows_a * KS);
        rsb = make_rsrc((const char*)p.SB + (int64_t)fc.tn * BN * KS, (uint32_t)rows_b * KS);
    };
    // offsets of the stream's slice (out of range past the last one: zeros)
    uint32_t foff0 = 0, soff = 0;
    const uint32_t sc_row = (uint32_t)((wave & 3) * 64 + lane) * KS;
    auto feed_offsets = [&](bool live) __attribute__((always_inline)) {
        foff0 = live ? cp_off + (uint32_t)(fc.kk * RB) : kOutOfRange;
        soff = live ? sc_row + (uint32_t)fc.kk * 16u : kOutOfRange;
    };
    int fg = 0;  // the copy stream's slice
    auto feed_next = [&]() __attribute__((always_inline)) {
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
    // copy c (0..17) of the stream's slice into stage / piece buffer st:
    // 0..15 elements, 16 and 17 the scale rows 64 q .. 64 q + 63 (q = wave,
    // wave + 4) of the A (q < 4) then B rows, 16 bytes per row and lane
    // element copy x (0..15) of the stream's slice into stage st: 1 KiB block
    // 4 (x % 8) + w of the A (x < 8) or B region, i.e. byte 4096 x + 1024 w
    auto copy_elements = [&](int st, int x) __attribute__((always_inline)) {
        copy16_to_lds(x < 8 ? ra : rb, lds + st * STAGE + x * 4096 + wave * 1024,
                      foff0 + (uint32_t)(x & 7) * cp_step);
    };
    // scale copy h of the stream's slice into piece buffer st: rows
    // 64 (w + 4 h) .. + 63 of the A (h = 0) or B (h = 1) rows
    auto copy_scales = [&](int st, int h) __attribute__((always_inline)) {
        copy16_to_lds(h == 0 ? rsa : rsb, scb + st * CHUNK + (wave + 4 * h) * 1024, soff);
    };

    // ---- fragments -----------------------------------------------------------
    // raw[f]: 8 bytes of fragment f (A blocks 0-7, then B blocks 8-15): half h
    // of logical chunk 4 q + l / 16 of row l % 16 of the block (quad q),
    // stored at chunk ^ ((row / 2) % 8), i.e. the 16 E2M1 values of block
    // 8 q + 2 (l / 16) + h of the slice; sc[f]: that block's E4M3 scale,
    // made fp16 at the half's first conversion; cv[f]: the fp16 fragment of
    // the current K step.  K step t of a slice takes half (t / 2 + l / 16) % 2
    // of quad t / 4, dword t % 2.
    const int r16 = lane & 15, g4 = lane >> 4;
    const int xr = r16 >> 1;
    const uint32_t a_row = (uint32_t)(wm * 128 + r16) * RB;
    const uint32_t b_row = (uint32_t)A_BYTES + (uint32_t)(wn * 128 + r16) * RB;
    const uint32_t chq0 = (uint32_t)((0 + g4) ^ xr) * 16u, chq1 = (uint32_t)((4 + g4) ^ xr) * 16u;
    const uint32_t sa_row = (uint32_t)(wm * 128 + r16) * 16u + 2u * (uint32_t)g4;
    const uint32_t sb_row = 4096u + (uint32_t)(wn * 128 + r16) * 16u + 2u * (uint32_t)g4;
    f32x4_t acc[8][8];
    i32x4_t cv[16];
    i32x2_t raw[16];
    int sc[16];
    // the half of each fragment read next: its offset in the ring (lane part
    // included) and in the scale piece buffers
    uint32_t nro = chq0, nso = 0;
    auto read_raw = [&](int f) __attribute__((always_inline)) {
        const uint32_t row = f < 8 ? a_row + (uint32_t)f * 16u * RB : b_row + (uint32_t)(f - 8) * 16u * RB;
        raw[f] = *(const i32x2_t*)(lds + nro + row);
        const uint32_t srow = f < 8 ? sa_row + (uint32_t)f * 256u : sb_row + (uint32_t)(f - 8) * 256u;
        sc[f] = *(const unsigned char*)(scb + nso + srow);
    };
    // the half that K steps 2 n and 2 n + 1 of slice h take (n = 0 .. 3)
    auto aim_reads = [&](int h, int n) __attribute__((always_inline)) {
        const int st = h & 1, q = n >> 1;
        const uint32_t hf = (uint32_t)((n ^ g4) & 1);
        nro = (uint32_t)(st * STAGE) + (q ? chq1 : chq0) + 8u * hf;
        nso = (uint32_t)(st * CHUNK + 8 * q) + hf;
    };
    // Part PP of fragment F for a K step of parity T (values 2 PP, 2 PP + 1 of
    // the lane's 8: byte PP of dword T of the half), in two stages one
    // product apart, so that neither waits for the other: the conversion into
    // ct[slot parity][j] (j: 0, 1 for the parts of slot x, 2, 3 for those of
    // slot x + 64; the half's scale made fp16 with the first part),
    // then the scale multiplication into cv.  (Inline assembly keeps each
    // stage after its product: as plain arithmetic the compiler gathers the
    // conversions into runs that stall the matrix core.)
    int ct[2][4];
    auto convert = [&](auto F, auto PP, auto T, auto SLOT, auto J) __attribute__((always_inline)) {
        constexpr int f = decltype(F)::value, pp = decltype(PP)::value, t = decltype(T)::value;
        constexpr int sl = decltype(SLOT)::value & 1, j = decltype(J)::value;
        ct[sl][j] = fp4_pair<pp, t == 0 && pp == 0>((uint32_t)raw[f][t], sc[f]);
    };
    auto scale = [&](auto F, auto PP, auto SLOT, auto J) __attribute__((always_inline)) {
        constexpr int f = decltype(F)::value, pp = decltype(PP)::value;
        constexpr int sl = decltype(SLOT)::value & 1, j = decltype(J)::value;
        cv[f][pp] = fp16x2_scaled<g16nv::conv_nops(f, pp)>(ct[sl][j], sc[f]);
    };
    auto mma = [&](int i, int j, f32x4_t c) __attribute__((always_inline)) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, cv[8 + j]),
                                                           __builtin_bit_cast(f16x8_t, cv[i]), c, 0, 0, 0);
    };
    // Conversion work after product x of K step S of a pair: first the scale
    // multiplications of the parts converted after product x - 1 (after a
    // last part for a pair's second K step, S = 1, the fragment's next half
    // is read), then the conversions of the parts whose slot is x (for the
    // next K step) or x + 64 (for this one).  PRO: the prologue, which
    // converts for the first K step only and has no product before its first.
    auto conversions = [&](auto S, auto X, auto PRO) __attribute__((always_inline)) {
        constexpr int sp = decltype(S)::value, x = decltype(X)::value;
        constexpr bool pro = decltype(PRO)::value;
        static_for<4>([&](auto Q) __attribute__((always_inline)) {
            constexpr int q = decltype(Q)::value;
            // previous slot: x - 1 (next / this K step), or 63 of the K step before
            constexpr bool next = q < 2;
            constexpr int ps = x > 0 ? (next ? x - 1 : x - 1 + 64) : (next ? 63 : 127);
            constexpr int code = g16nv::task_at(ps, q & 1);
            if constexpr (code >= 0 && !(pro && x == 0) && (next || !pro)) {
                constexpr int f = code >> 2, pp = code & 3;
                // parity of the K step served: from the step before (x == 0) it is this one
                constexpr int par = x > 0 ? (next ? 1 - sp : sp) : sp;
                scale(std::integral_constant<int, f>{}, std::integral_constant<int, pp>{},
                      std::integral_constant<int, ps>{}, std::integral_constant<int, q>{});
                if constexpr (pp == 3 && par == 1) read_raw(f);
            }
        });
        static_for<4>([&](auto Q) __attribute__((always_inline)) {
            constexpr int q = decltype(Q)::value;
            constexpr bool next = q < 2;  // slot x: for the next K step; slot x + 64: for this one
            constexpr int slot = next ? x : x + 64;
            constexpr int code = g16nv::task_at(slot, q & 1);
            if constexpr (code >= 0 && (next || !pro)) {
                constexpr int f = code >> 2, pp = code & 3;
                constexpr int par = next ? 1 - sp : sp;  // parity of the K step served
                convert(std::integral_constant<int, f>{}, std::integral_constant<int, pp>{},
                        std::integral_constant<int, par>{}, std::integral_constant<int, slot>{},
                        std::integral_constant<int, q>{});
            }
        });
    };

    // ---- epilogue --------------------------------------------------------------
    const float alpha = p.alpha;
    auto epilogue = [&](const TileCursor& c) __attribute__((always_inline)) {
        const int ldc = p.N;
        char* Cb = (char*)p.C + c.batch * p.stride_c;
        const int m0 = c.tm * BM + wm * 128, n0 = c.tn * BN + wn * 128;
        const bool full = c.tm * BM + BM <= p.M && c.tn * BN + BN <= p.N;
        if (STG_ROWS > 0 && full && ldc % (16 / (int)sizeof(TOut)) == 0) {
            constexpr int CHK = STG_ROWB / 16;
            constexpr int RPI = kWaveSize * 16 / STG_ROWB;
            char* stg = lds + S * STAGE + SC_BYTES + wave * STG_BYTES;
            const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
            const int rr = ln & 15, gg = ln >> 4;
#pragma unroll
            for (int ps = 0; ps < (STG_ROWS > 0 ? 8 : 0); ++ps) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const f32x4_t v = acc[ps][j] * alpha;
                    const int byte = (16 * j + 4 * gg) * (int)sizeof(TOut);
                    const int chunk = (byte / 16) ^ rr;
                    store4<TOut>((TOut*)(stg + rr * STG_ROWB + chunk * 16 + byte % 16), v[0], v[1], v[2],
                                 v[3]);
                }
                wave_lds_exchange();
#pragma unroll
                for (int t = 0; t < (STG_ROWS > 0 ? STG_ROWS / RPI : 0); ++t) {
                    const int r = t * RPI + ln / CHK;
                    const int ck = ln % CHK;
                    const i32x4_t d = *(const i32x4_t*)(stg + r * STG_ROWB + ((ck ^ (r & 15)) * 16));
                    char* gp =
                        Cb + ((int64_t)(m0 + 16 * ps + r) * ldc + n0) * (int64_t)sizeof(TOut) + ck * 16;
                    __builtin_nontemporal_store(d, (i32x4_t*)gp);
                }
                wave_lds_exchange();
            }
            return;
        }
        // edge tile, fp32 output, or rows not 16-byte aligned: rows past M and
        // columns past N are not written
        const bool vec = (ldc & 3) == 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int m = m0 + 16 * i + r16;
            if (m >= p.M) continue;
            TOut* row = (TOut*)Cb + (int64_t)m * ldc;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int n = n0 + 16 * j + 4 * g4;
                const f32x4_t v = acc[i][j] * alpha;
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

    // ---- two K steps: 2 n and 2 n + 1 of slice g (ZERO: the tile's first
    // pair, whose products start from zero).  Pair 3 opens with the hand-off;
    // every pair carries one copy group of the stream's slice fg (slice
    // g + 2 in pair 3, g + 1 in pairs 0-2), into stage fg % 2.
    auto pair = [&](int g, int n, auto ZERO) __attribute__((always_inline)) {
        aim_reads(n == 3 ? g + 1 : g, (n + 1) & 3);
        // this pair's copy group: resource, LDS block of its first copy, offset
        const int cq = (n + 1) & 3;
        const __amdgpu_buffer_rsrc_t ce = cq < 2 ? ra : rb;
        char* const cdst = lds + (fg & 1) * STAGE + cq * 4 * 4096 + wave * 1024;
        const uint32_t coff = foff0 + (uint32_t)(4 * (cq & 1)) * cp_step;
        static_for<2>([&](auto S) __attribute__((always_inline)) {
            constexpr int sp = decltype(S)::value;
            static_for<64>([&](auto X) __attribute__((always_inline)) {
                constexpr int x = decltype(X)::value;
                constexpr int i = g16::a_of(x), j = g16::b_of(x);
                mma(i, j, decltype(ZERO)::value && sp == 0 ? (f32x4_t){} : acc[i][j]);
                if constexpr (sp == 0 && x == 0) {
                    if (n == 3) {
                        wait_vmcnt<0>();
                        barrier_lds();
                    }
                }
                constexpr int k = g16nv::copy_at(x);
                if constexpr (sp == 0 && k >= 0) {
                    copy16_to_lds(ce, cdst + k * 4096, coff + (uint32_t)k * cp_step);
                    if constexpr (k == 3) {
                        if (n == 2) feed_next();
                    }
                }
                if constexpr (sp == 1 && x == g16nv::kScaleCopySlot) {
                    if (cq < 2) copy_scales(fg & 1, cq);
                }
                conversions(S, X, std::false_type{});
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };

    // ---- prologue: slice 0 whole, copy group 0 of slice 1, the fragments of
    // slice 0's first K step -------------------------------------------------
    locate(fc);
    feed_resources();
    feed_offsets(true);
#pragma unroll
    for (int x = 0; x < 16; ++x) copy_elements(0, x);
    copy_scales(0, 0);
    copy_scales(0, 1);
    feed_next();
#pragma unroll
    for (int x = 0; x < 4; ++x) copy_elements(1, x);
    copy_scales(1, 0);
    wait_vmcnt<5>();  // (slice 0)
    barrier_lds();
    aim_reads(0, 0);
#pragma unroll
    for (int f = 0; f < 16; ++f) read_raw(f);
    // the parts that the second K step of a preceding pair would have converted
    static_for<64>([&](auto X) __attribute__((always_inline)) {
        conversions(std::integral_constant<int, 1>{}, X, std::true_type{});
    });

    int g0 = 0;  // the tile's first slice
    for (int tl = 0; tl < my_tiles; ++tl) {
        pair(g0, 0, std::true_type{});
        for (int k = 1; k < 4 * p.ksteps; ++k) pair(g0 + (k >> 2), k & 3, std::false_type{});
        g0 += p.ksteps;
        TileCursor ec = {tl, 0, 0, 0, 0};
        locate(ec);
        __builtin_amdgcn_sched_barrier(0);
        epilogue(ec);
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace tcm
