// The tiled product kernel for gfx950: Out = A . B^T, A M x K and B N x K
// both K-contiguous ("TN"), fp32 accumulation in the matrix cores.  For
// 16-bit inputs either operand may instead be stored with its M (N) index
// contiguous, K rows of M (N) values ("API Card: Blackwell Pipeline
// (tcgen05)", Descriptor: half and bfloat16 run in either majorness), and
// every operand, the C input and the output take a leading dimension.
//
// Structure (the pipelined tile loop of "Hopper and Blackwell GEMM", Concept
// and Maths sections, and of "API Card: Blackwell Pipeline (tcgen05)",
// Device side., rebuilt for CDNA4):
//
//  * Persistent tile scheduler.  A workgroup takes output tiles
//    lid, lid + G, lid + 2G, ... of a host-computed tile count, with an
//    XCD-aware renumbering of workgroups and a grouped tile order; every wave
//    of the workgroup leaves the loop at the same point.
//  * One flattened loop over (tile, K slice) pairs, g = t * ksteps + k, as in
//    the page's slice numbering.  Operand copies run S - 1 slices ahead of the
//    matrix cores, across tile boundaries, so the next tile's first slices are
//    already in flight while the current tile's epilogue converts and stores.
//  * LDS ring of S stages, one A tile and one B tile per stage.  Copies go
//    from HBM straight into LDS (buffer_load ... lds, 16 bytes per lane),
//    without passing through registers; out-of-range rows and the K tail read
//    as zeros through the buffer resource's bounds.
//  * Stage hand-off: the "full" condition is this wave's own vmcnt wait plus
//    the workgroup barrier; the "empty" condition is the same barrier, since
//    every wave has read its fragments of the previous slice before it.
//  * XOR-swizzled LDS rows so that each group of 16 lanes of a 16-byte
//    fragment read spreads over all 64 banks (the swizzled shared layouts of "Blackwell Tensor
//    Cores", The Accumulator's Lifetime, redesigned for LDS banks).
//  * Four waves in a 2 x 2 arrangement, each owning a (BM/2) x (BN/2) block of
//    32 x 32 MFMA accumulators; the first slice of a tile starts from zero and
//    later slices accumulate ("mma.sync", Code generation: the first K issue
//    reads C, later issues read D).
//  * Epilogue: fp32 accumulators converted (bf16 round-to-nearest-even, or
//    fp32 as is) and stored with edge masks.
#pragma once

#include <type_traits>

#include "tcm_device.h"

namespace tcm {

// ---------------------------------------------------------------------------
// Matrix-core operations.  The 32x32 MFMA forms take, per lane l, operand row
// l % 32 and one contiguous run of K values selected by l / 32; the result
// lands as 16 floats per lane: rows 8*(r/4) + 4*(l/32) + r%4, column l % 32.
// ---------------------------------------------------------------------------
struct OpBF16 {
    static constexpr int kElemBytes = 2;
    static constexpr bool kNV4 = false;
    static constexpr int kElemBits = 16;
    static constexpr int kK = 16;  // K per MFMA
    static constexpr bool kScaled = false;
    typedef bf16x8_t frag_t;
    __device__ static __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

struct OpF16 {
    static constexpr int kElemBytes = 2;
    static constexpr bool kNV4 = false;
    static constexpr int kElemBits = 16;
    static constexpr int kK = 16;
    static constexpr bool kScaled = false;
    typedef f16x8_t frag_t;
    __device__ static __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// MXFP8: E4M3 x E4M3 with one E8M0 scale per 32 K values per row, applied by
// the scaled MFMA.  Of the 64 K values of one MFMA, block 0 sits in bytes
// 0..15 of lanes l and l + 32 and block 1 in bytes 16..31; lane l + 32 b
// supplies the scale of block b of row l % 32.  `SEL` picks the byte of the
// 32-bit scale register.
struct OpMXFP8 {
    static constexpr int kElemBytes = 1;
    static constexpr bool kNV4 = false;
    static constexpr int kElemBits = 8;
    static constexpr int kK = 64;
    static constexpr bool kScaled = true;
    typedef i32x8_t frag_t;
    template <int SEL>
    __device__ static __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c, int sa, int sb) {
        // format codes 0 / 0: both operands FP8 E4M3
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, sa, SEL, sb);
    }
};

// MXFP4: E2M1 x E2M1, two elements per byte (element 2t in the low four
// bits of byte t), one E8M0 scale per 32 K values.  The scaled MFMA reads the
// first four registers of each operand, and (unlike FP8) lane l + 32 b holds
// the whole block b of row l % 32: 32 K values in 16 bytes, together with
// that block's scale.  Established on the device by feeding one nonzero
// element per lane with block scales 1 and 2: every nibble of lanes 0..31
// took scale 1, every nibble of lanes 32..63 scale 2.
struct OpMXFP4 {
    static constexpr int kElemBytes = 0;  // two elements per byte
    static constexpr bool kNV4 = false;
    static constexpr int kElemBits = 4;
    static constexpr int kK = 64;
    static constexpr bool kScaled = true;
    typedef i32x4_t frag_t;
    template <int SEL>
    __device__ static __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c, int sa, int sb) {
        const i32x8_t a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
        const i32x8_t b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);
        // format codes 4 / 4: both operands FP4 E2M1
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, SEL, sa, SEL, sb);
    }
};

// MXFP6: E2M3 (format code 2) or E3M2 (code 3) x the same, one E8M0 scale
// per 32 K values.  Like FP4, lane l + 32 b holds the whole block b of row
// l % 32: 32 six-bit codes in six registers, code t in bits 6t .. 6t + 5 of
// their little-endian concatenation -- the same bit stream as the packed
// storage, so a block is its 24 stored bytes.  (Established on the device:
// with block scales 1 and 2 on A and 1 and 4 on B, a 1.0 in any of the 32
// slots of a lane of half-wave b scaled by block b's scales.)
template <int FMT>
struct OpMXFP6 {
    static constexpr int kElemBytes = 0;
    static constexpr bool kNV4 = false;
    static constexpr int kElemBits = 6;
    static constexpr int kK = 64;
    static constexpr bool kScaled = true;
    typedef i32x8_t frag_t;  // registers 0..5 used
    template <int SEL>
    __device__ static __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c, int sa, int sb) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, SEL, sa, SEL, sb);
    }
};

// NVFP4 (E2M1 with an E4M3 scale per 16 and an fp32 scale per tensor).  No
// matrix-core form takes E4M3 block scales, but an E2M1 value times an E4M3
// scale is exact in fp16 (at most 6 significant bits, magnitudes 2^-10 ..
// 2688): the copies dequantize into the fp16 LDS tile and the product runs on
// the fp16 MFMA; the tensor scales enter as the epilogue's alpha.  WIDE: a
// row's scales of four slices come in one 16-byte load (K a multiple of 256,
// scale rows 16-byte aligned); otherwise two bytes per half row and slice.
template <bool WIDE>
struct OpNVFP4 {
    static constexpr bool kWide = WIDE;
    static constexpr int kElemBytes = 2;  // of the LDS tile (fp16)
    static constexpr int kElemBits = 16;
    static constexpr bool kNV4 = true;
    static constexpr int kK = 16;
    static constexpr bool kScaled = false;
    typedef f16x8_t frag_t;
    __device__ static __forceinline__ f32x16_t mma(frag_t a, frag_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <class Op>
constexpr bool nv4_wide() {
    if constexpr (Op::kNV4)
        return Op::kWide;
    else
        return false;
}

struct TileCursor {
    int tl, kk, batch, tm, tn;
};

// VG selects the copy path: false, direct-to-LDS DMA (`buffer_load ... lds`);
// true, 16-byte buffer loads into registers one slice ahead and `ds_write_b128`
// into the ring when the stage is free (plain bf16/f16, 2-stage ring).
// AB builds the epilogue with a C input: Out = alpha * (A B^T) + beta * C,
// combined in fp32 in the accumulator layout and rounded once to TOut.
// A_MN (B_MN): A (B) is stored M-major (N-major): K rows of lda (ldb)
// elements, the tile's BM (BN) values of one k contiguous.  DENSE: both
// operands K-major with rows K apart and Out's rows N apart; the kernel then
// ignores the leading dimensions, so one register holds the copy offsets of
// both operands and no argument register is added (the 256 x 256 kernels
// with the LDS-staged epilogue have none to spare: one more spills).
template <class Op, typename TOut, int BM, int BN, int BK, int S, int OCC, int SWZ,
          bool SCALE_WORDS = false, int NSPLIT = 1, bool EPI_LDS = false, bool VG = false,
          bool AB = false, bool A_MN = false, bool B_MN = false, bool DENSE = true>
__global__ __launch_bounds__(kThreads, OCC) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void tiled_gemm_kernel(GemmArgs p) {
    constexpr int ESZ = Op::kElemBytes;
    constexpr int RB = BK * ESZ;   // bytes of one operand row's K slice
    constexpr int CPR = RB / 16;   // 16-byte chunks per row
    constexpr int A_BYTES = BM * RB;
    constexpr int B_BYTES = BN * RB;
    constexpr int STAGE = A_BYTES + B_BYTES;
    // NVFP4: a copy ("task") is one row's 64-element slice: task x of thread
    // tid is row tid + 256 x of the A tile stacked on the B tile.  A wave's
    // 64 rows lie in one operand, so the operand choice is wave-uniform.
    constexpr bool NV4 = Op::kNV4;
    constexpr int A_LOADS = NV4 ? 0 : A_BYTES / (kThreads * 16);  // DMA copies per thread per slice
    constexpr int B_LOADS = NV4 ? 0 : B_BYTES / (kThreads * 16);
    constexpr int ROWS_PER_WAVE_COPY = kWaveSize * 16 / RB;
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int KSTEPS = BK / Op::kK;
    constexpr int CPL = Op::kK * ESZ / 32;  // 16-byte chunks per lane per MFMA
    constexpr int LOADS = NV4 ? (BM + BN) / kThreads : A_LOADS + B_LOADS;
    static_assert(KSTEPS % 2 == 0, "fragment double buffer alternates per K step");
    static_assert(((4 * ROWS_PER_WAVE_COPY) >> SWZ) % CPR == 0, "copy chunk independent of i");
    static_assert((S - 1) * LOADS < 64, "vmcnt range");
    static_assert(NSPLIT >= 1 && NSPLIT <= KSTEPS && NSPLIT <= LOADS, "copy split");
    // Part p of a slice's copies: copies part_base(p) .. part_base(p + 1) - 1.
    // Uneven splits put the larger parts first (16 copies in 3 parts: 6/5/5),
    // since an earlier part has longer to land before the next hand-off
    // (measured +1 % over 5/5/6 on the bf16 256 x 256 kernel).
    auto part_base = [](int p) { return (p * LOADS + NSPLIT - 1) / NSPLIT; };
    constexpr int PART = (LOADS + NSPLIT - 1) / NSPLIT;  // copies in part 0 (the largest)
    constexpr int PMAX = PART;                           // largest part
    static_assert(CPR == 4 || CPR == 8, "row slice must be 64 or 128 bytes");
    static_assert(A_BYTES % (kThreads * 16) == 0 && B_BYTES % (kThreads * 16) == 0, "copy split");
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert(S >= 2, "ring depth");
    static_assert((32 >> SWZ) % CPR == 0, "swizzle must depend on the row within 32 only");
    static_assert(!Op::kScaled || (BK == 128 && S == 2), "MX path: 128-deep slices, 2 stages");
    static_assert(!VG || (!Op::kScaled && S == 2), "register-staged copies: plain types, 2 stages");
    static_assert(!NV4 || (VG && BK == 64 && BM % kWaveSize == 0 && (BM + BN) % kThreads == 0),
                  "NVFP4: register-staged copies of 64-deep slices, whole rows per thread");
    static_assert(Op::kElemBits >= 8, "whole-byte elements");
    constexpr bool ANY_MN = A_MN || B_MN;
    static_assert(!ANY_MN || (!VG && ((ESZ == 2 && !Op::kScaled) || (ESZ == 1 && Op::kScaled && CPL == 2))),
                  "M/N-major: 16-bit or MXFP8, DMA copies");
    static_assert(!(DENSE && ANY_MN), "dense storage: both operands K-major");
    static_assert((!A_MN || BM * ESZ >= (ESZ == 2 ? 256 : 128)) &&
                      (!B_MN || BN * ESZ >= (ESZ == 2 ? 256 : 128)),
                  "M/N-major rows of at least 16 chunks (16-bit) or 8 chunks (8-bit): bank "
                  "spread of the transposing reads");

    // Epilogue staging: one 32-row block of a wave's output at a time, in a
    // wave-private LDS area after the ring.
    constexpr int STG_ROWB = WTN * (int)sizeof(TOut);  // bytes of one staged row
    constexpr int STG_BYTES = EPI_LDS ? 32 * STG_ROWB : 0;
    // C-input kernels: an fp32 staging area per wave for the epilogue with a
    // per-element operation, 32 rows of OPJ 32-column accumulator blocks, as
    // many blocks as the workgroups of one CU leave room for (0: the tile
    // has no room, and the host never asks it for an operation).
    constexpr int OPJ = !AB ? 0
                        : (FN % 4 == 0 && OCC * (S * STAGE + 4 * 32 * 128 * 4) <= 160 * 1024) ? 4
                        : (FN % 2 == 0 && OCC * (S * STAGE + 4 * 32 * 64 * 4) <= 160 * 1024)  ? 2
                        : (OCC * (S * STAGE + 4 * 32 * 32 * 4) <= 160 * 1024)                 ? 1
                                                                                              : 0;
    constexpr int OP_BYTES = 32 * OPJ * 32 * 4;  // per wave
    constexpr int EPI_BYTES = 4 * (STG_BYTES > OP_BYTES ? STG_BYTES : OP_BYTES);
    static_assert(S * STAGE + EPI_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char lds[S * STAGE + EPI_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, hi = lane >> 5;

    const int G = gridDim.x;
    const int lid = logical_block(blockIdx.x, G);
    if (lid >= p.total_tiles) return;
    const int my_tiles = (p.total_tiles - 1 - lid) / G + 1;
    const int total = my_tiles * p.ksteps;
    const int K = p.K;

    // ---- per-lane copy geometry -------------------------------------------
    // K-major operand: copy i of wave w fills LDS chunk q = (4 i + w) * 64 +
    // lane of the A (B) region: row q / CPR, physical chunk q % CPR, which
    // holds logical chunk (q % CPR) ^ swz(row) of that row's K slice.  The
    // chunk is the same for every i, and copy i sits 4 * ROWS_PER_WAVE_COPY
    // rows below copy i - 1.
    const int cp_row = wave * ROWS_PER_WAVE_COPY + lane / CPR;
    const int cp_chunk = (lane % CPR) ^ ((cp_row >> SWZ) & (CPR - 1));
    const int cp_k = cp_chunk * (16 / ESZ);  // first K element of the chunk
    // M-major (N-major) operand: the region holds BK rows, one per k of the
    // slice, of the tile's BM (BN) values; chunk q is row q / cpr, physical
    // chunk q % cpr, holding logical chunk (q % cpr) ^ swz(row), so that the
    // rows a transposing read touches sit in different bank groups: 16-bit
    // reads cover 4 rows (swz = 4 (row % 4)); 8-bit reads cover 8 rows, with
    // the neighbouring 16-lane group on the next chunk (swz = 2 (row % 8) for
    // rows of 16 or more chunks; 2 ((row / 2) % 4) for rows of 8 chunks,
    // where two rows share a 256-byte bank line).
    auto mn_swz = [](int row, int cpr) {
        return ESZ == 2 ? 4 * (row & 3) : cpr >= 16 ? 2 * (row & 7) : 2 * ((row >> 1) & 3);
    };
    struct CopyGeo {
        uint32_t off, step;  // buffer offset of copy 0, and from copy i to i + 1
    };
    auto kmajor_geo = [&](int ld) -> CopyGeo {
        return {(uint32_t)cp_row * (uint32_t)ld * ESZ + cp_chunk * 16,
                4u * ROWS_PER_WAVE_COPY * (uint32_t)ld * ESZ};
    };
    auto mn_geo = [&](int rows, int ld) -> CopyGeo {
        const int cpr = rows * ESZ / 16, rpw = kWaveSize / cpr;
        const int row = wave * rpw + lane / cpr;
        const int ch = (lane % cpr) ^ mn_swz(row, cpr);
        return {(uint32_t)row * (uint32_t)ld * ESZ + ch * 16, 4u * rpw * (uint32_t)ld * ESZ};
    };
    const int lda = DENSE ? K : p.lda;
    const int ldb = DENSE ? K : p.ldb;
    const CopyGeo geo_a = A_MN ? mn_geo(BM, lda) : kmajor_geo(lda);
    const CopyGeo geo_b = B_MN ? mn_geo(BN, ldb) : kmajor_geo(ldb);

    auto locate = [&](TileCursor& c) {
        tile_coords(p, c.tl * G + lid, c.batch, c.tm, c.tn);
    };
    auto advance = [&](TileCursor& c) {
        if (++c.kk == p.ksteps) {
            c.kk = 0;
            if (++c.tl < my_tiles) locate(c);
        }
    };

    // The copy stream ("producer"): the next slice to copy and the buffer
    // resources of its tile, rebuilt when the stream enters a new tile (and,
    // with an M/N-major operand, at every slice).
    TileCursor fc = {0, 0, 0, 0, 0};
    __amdgpu_buffer_rsrc_t ra, rb;
    __amdgpu_buffer_rsrc_t rsa, rsb;  // NVFP4 block scales
    // K-major: the tile's rows r0 .. r0 + rows - 1; rows past the tile's last
    // (r >= rows) start at or beyond the bound.
    auto kmajor_rsrc = [&](const char* base, int r0, int R, int BR, int ld) {
        const int rows = min(BR, R - r0);
        return make_rsrc(base + (int64_t)r0 * ld * ESZ, (uint32_t)((rows - 1) * ld + K) * ESZ);
    };
    // M/N-major: k rows k0 .. k0 + kv - 1 of the slice, columns r0 .. r0 + BR - 1;
    // the bound ends with the last row's last 16-byte piece that holds a
    // valid column (ld is a whole number of pieces: a multiple of 8 16-bit
    // or 16 8-bit elements), so rows past K read as zeros and no read leaves
    // the operand's storage.
    auto mn_rsrc = [&](const char* base, int r0, int R, int BR, int ld, int k0) {
        constexpr int EPC = 16 / ESZ;  // elements per 16-byte piece
        const int kv = min(BK, K - k0);
        const int cols = min(BR, ((R + EPC - 1) & ~(EPC - 1)) - r0);
        const uint32_t bytes = kv > 0 ? (uint32_t)((kv - 1) * ld + cols) * ESZ : 0u;
        return make_rsrc(base + ((int64_t)k0 * ld + r0) * ESZ, bytes);
    };
    auto feed_resources = [&]() {
        const char* abase = (const char*)p.A + fc.batch * p.stride_a;
        const char* bbase = (const char*)p.B + fc.batch * p.stride_b;
        if constexpr (NV4) {
            // rows of K/2 bytes of E2M1 pairs and of K/16 E4M3 scales
            const int rows_a = min(BM, p.M - fc.tm * BM), rows_b = min(BN, p.N - fc.tn * BN);
            ra = make_rsrc(abase + (int64_t)fc.tm * BM * (K / 2), (uint32_t)rows_a * (K / 2));
            rb = make_rsrc(bbase + (int64_t)fc.tn * BN * (K / 2), (uint32_t)rows_b * (K / 2));
            rsa = make_rsrc((const char*)p.SA + (int64_t)fc.tm * BM * (K / 16),
                            (uint32_t)rows_a * (K / 16));
            rsb = make_rsrc((const char*)p.SB + (int64_t)fc.tn * BN * (K / 16),
                            (uint32_t)rows_b * (K / 16));
            return;
        }
        if constexpr (A_MN)
            ra = mn_rsrc(abase, fc.tm * BM, p.M, BM, lda, fc.kk * BK);
        else
            ra = kmajor_rsrc(abase, fc.tm * BM, p.M, BM, lda);
        if constexpr (B_MN)
            rb = mn_rsrc(bbase, fc.tn * BN, p.N, BN, ldb, fc.kk * BK);
        else
            rb = kmajor_rsrc(bbase, fc.tn * BN, p.N, BN, ldb);
    };
    auto feed_advance = [&]() {
        if (++fc.kk == p.ksteps) {
            fc.kk = 0;
            if (++fc.tl < my_tiles) {
                locate(fc);
                feed_resources();
            }
        } else if constexpr (ANY_MN) {
            feed_resources();
        }
    };
    // Buffer offsets of copy 0 of the stream's current slice, computed
    // outside the hot region; copy i adds i * step.  A slice past the last
    // one (`live` false) and K-major 16-byte chunks past K get out-of-range
    // offsets (>= 2^31, beyond any tile's records even after adding
    // i * step): those copies touch no memory and write zeros into a stage
    // that is never read again.  (An M/N-major slice's resource starts at
    // its own first k row, so its offsets do not move with k.)
    uint32_t foff_a0, foff_b0;
    int nv_k0 = -1;  // NVFP4: first K element of the stream's slice, -1 past the last one
    auto feed_offsets = [&](bool live) {
        if constexpr (NV4) {
            nv_k0 = live ? fc.kk * BK : -1;
            return;
        }
        const uint32_t k0b = (uint32_t)(fc.kk * BK) * ESZ;
        const bool kin = fc.kk * BK + cp_k < K;
        foff_a0 = A_MN ? (live ? geo_a.off : kOutOfRange)
                       : (live && kin ? geo_a.off + k0b : kOutOfRange);
        if constexpr (!DENSE)
            foff_b0 = B_MN ? (live ? geo_b.off : kOutOfRange)
                           : (live && kin ? geo_b.off + k0b : kOutOfRange);
    };
    auto foff_a = [&](int i) -> uint32_t { return foff_a0 + (uint32_t)i * geo_a.step; };
    auto foff_b = [&](int i) -> uint32_t {
        if constexpr (DENSE)
            return foff_a(i);
        else
            return foff_b0 + (uint32_t)i * geo_b.step;
    };
    // One 16-byte copy per lane; kernels with transposing reads issue it in
    // the assembly form (see copy16_to_lds_asm).
    auto dma = [&](__amdgpu_buffer_rsrc_t r, char* dst, uint32_t off) {
        if constexpr (ANY_MN)
            copy16_to_lds_asm(r, dst, off);
        else
            copy16_to_lds(r, dst, off);
    };
    // Copies of the stream's current slice into ring stage `st`.
    auto issue = [&](int st) {
        char* sa = lds + st * STAGE;
        char* sb = sa + A_BYTES;
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) dma(ra, sa + (4 * i + wave) * 1024, foff_a(i));
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) dma(rb, sb + (4 * i + wave) * 1024, foff_b(i));
    };

    // ---- per-lane fragment geometry ---------------------------------------
    const int xr = (l32 >> SWZ) & (CPR - 1);
    const uint32_t a_frag = (uint32_t)(wm * WTM + l32) * RB;
    const uint32_t b_frag = (uint32_t)A_BYTES + (uint32_t)(wn * WTN + l32) * RB;

    typedef typename Op::frag_t frag_t;
    auto read_frag = [&](const char* base, int s) -> frag_t {
        frag_t f;
        if constexpr (CPL == 1) {
            int ch = (2 * s + hi) ^ xr;
            f = *(const frag_t*)(base + ch * 16);
        } else {
            // 64 K values per MFMA form two scale blocks of 32.  The scaled
            // MFMA takes block 0 from bytes 0..15 of both half-waves and block
            // 1 from bytes 16..31, so half-wave h reads K chunks h and 2 + h.
            int ch0 = (4 * s + hi) ^ xr;
            int ch1 = (4 * s + 2 + hi) ^ xr;
            i32x4_t lo = *(const i32x4_t*)(base + ch0 * 16);
            i32x4_t up = *(const i32x4_t*)(base + ch1 * 16);
            f = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        return f;
    };
    // M-major (N-major) regions: transposing reads.  For fragment block f
    // and K step s, lane 16 g + t reads the 8 bytes at k row
    // 16 s + 8 (g / 2) + t / 4 (and 4 rows further for the second half),
    // columns c + 16 (g % 2) + 4 (t % 4) .. + 3, c the block's first column;
    // it receives k 16 s + 8 (g / 2) + 0..3 (4..7) of column
    // c + 16 (g % 2) + t, which is the MFMA operand layout (row l % 32,
    // K values 8 (l / 32) .. + 7).  k % 4 = t / 4 for every such read, so the
    // row's chunk swizzle is a per-lane constant folded into the offset.
    //
    // 8-bit (MXFP8) regions: ds_read_b64_tr_b8 gives lane t of a 16-lane
    // group byte t of each of the 8 rows its group addresses (row r from
    // lanes 2r and 2r + 1, bytes 0..7 and 8..15; probed on the device).  The
    // scaled MFMA wants, in lane l of half-wave h, row l % 32 with bytes
    // 0..15 = k 16 h .. 16 h + 15 and bytes 16..31 = k 32 + 16 h .. + 15, so
    // four reads (k offsets 0, 8, 32, 40) fill its 32 bytes: lane 16 g + t
    // reads k row 64 s + off + 16 (g / 2) + t / 2, columns
    // c + 16 (g % 2) + 8 (t % 2) .. + 7; k % 8 = t / 2, so the row's swizzle
    // is again a per-lane constant.
    const int g16 = lane >> 4, t16 = lane & 15;
    auto mn_frag_off = [&](int rowb, int col_byte) -> uint32_t {
        if constexpr (ESZ == 1)
            return (uint32_t)((16 * (g16 >> 1) + (t16 >> 1)) * rowb +
                              (col_byte ^ (16 * mn_swz(t16 >> 1, rowb / 16))) + 16 * (g16 & 1) +
                              8 * (t16 & 1));
        else
            return (uint32_t)((8 * (g16 >> 1) + (t16 >> 2)) * rowb + (col_byte ^ (64 * (t16 >> 2))) +
                              32 * (g16 & 1) + 8 * (t16 & 3));
    };
    constexpr int RBA = BM * ESZ, RBB = BN * ESZ;  // bytes of one k row, M/N-major regions
    uint32_t a_mn[A_MN ? FM : 1], b_mn[B_MN ? FN : 1];
    if constexpr (A_MN) {
#pragma unroll
        for (int i = 0; i < FM; ++i) a_mn[i] = mn_frag_off(RBA, (wm * WTM + 32 * i) * ESZ);
    }
    if constexpr (B_MN) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
            b_mn[j] = (uint32_t)A_BYTES + mn_frag_off(RBB, (wn * WTN + 32 * j) * ESZ);
    }
    auto read_frag_tr = [&](const char* at, int rowb) -> frag_t {
        if constexpr (ANY_MN && ESZ == 1) {
            const i32x2_t q0 = lds_read_tr8(at);
            const i32x2_t q1 = lds_read_tr8(at + 8 * rowb);
            const i32x2_t q2 = lds_read_tr8(at + 32 * rowb);
            const i32x2_t q3 = lds_read_tr8(at + 40 * rowb);
            const i32x4_t lo = __builtin_shufflevector(q0, q1, 0, 1, 2, 3);
            const i32x4_t up = __builtin_shufflevector(q2, q3, 0, 1, 2, 3);
            return __builtin_bit_cast(frag_t, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        } else if constexpr (ANY_MN) {
            const s16x4_t lo = lds_read_tr16(at);
            const s16x4_t up = lds_read_tr16(at + 4 * rowb);
            return __builtin_bit_cast(frag_t,
                                      __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            return frag_t{};
        }
    };
    // k rows of one K step: Op::kK (16 for the 16-bit MFMA, 64 for MXFP8)
    auto frag_a = [&](const char* st, int i, int s) -> frag_t {
        if constexpr (A_MN)
            return read_frag_tr(st + a_mn[i] + Op::kK * s * RBA, RBA);
        else
            return read_frag(st + a_frag + i * 32 * RB, s);
    };
    auto frag_b = [&](const char* st, int j, int s) -> frag_t {
        if constexpr (B_MN)
            return read_frag_tr(st + b_mn[j] + Op::kK * s * RBB, RBB);
        else
            return read_frag(st + b_frag + j * 32 * RB, s);
    };

    frag_t fa[2][FM], fb[2][FN];
    auto read_frags = [&](int buf, const char* st, int s) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = frag_a(st, i, s);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = frag_b(st, j, s);
    };

    // ---- MX scales: one 32-bit register per fragment row per slice; byte 0
    // holds block (k0/32 + hi), byte 2 block (k0/32 + 2 + hi), so the MFMA of
    // K step s selects byte 2 s.
    int sc_a[Op::kScaled ? FM : 1], sc_b[Op::kScaled ? FN : 1];
    int nx_a[Op::kScaled ? FM : 1], nx_b[Op::kScaled ? FN : 1];
    auto load_scales = [&](const TileCursor& c, int* out_a, int* out_b) {
        if constexpr (Op::kScaled) {
            const int kblocks = K / 32;
            const int kb0 = c.kk * (BK / 32);
#pragma unroll
            for (int f = 0; f < FM + FN; ++f) {
                const bool is_a = f < FM;
                const int idx = is_a ? f : f - FM;
                const int lim = is_a ? p.M : p.N;
                int row = (is_a ? c.tm * BM + wm * WTM : c.tn * BN + wn * WTN) + idx * 32 + l32;
                row = min(row, lim - 1);
                const uint8_t* src = (const uint8_t*)(is_a ? p.SA : p.SB) + (int64_t)row * kblocks;
                int v;
                if constexpr (SCALE_WORDS) {
                    uint32_t w = *(const uint32_t*)(src + kb0);
                    v = (int)(w >> (8 * hi));
                } else {
                    int q0 = kb0 + hi, q2 = kb0 + 2 + hi;
                    int b0 = q0 < kblocks ? src[q0] : 127;
                    int b2 = q2 < kblocks ? src[q2] : 127;
                    v = b0 | (b2 << 16);
                }
                if (is_a) out_a[idx] = v; else out_b[idx] = v;
            }
        }
    };

    // Accumulators hold D = B_frag . A_frag^T per 32 x 32 block (operands
    // swapped), so lane l owns output row m = l % 32 and, for each r / 4, the
    // four consecutive output columns 8 (r / 4) + 4 (l / 32) + 0..3.
    f32x16_t acc[FM][FN];
    // ZERO (a std::integral_constant) selects the first MFMA of a tile, which
    // takes an all-zero accumulator input instead of clearing the registers.
    // Single-element forms of the three streams of a K step.
    auto mma_one = [&](int buf, int s, int x, auto ZERO) {
        const int i = x / FN, j = x % FN;
        f32x16_t c;
        if constexpr (decltype(ZERO)::value)
            c = (f32x16_t){};
        else
            c = acc[i][j];
        if constexpr (Op::kScaled) {
            if (s == 0)
                acc[i][j] = Op::template mma<0>(fb[buf][j], fa[buf][i], c, sc_b[j], sc_a[i]);
            else
                acc[i][j] = Op::template mma<2>(fb[buf][j], fa[buf][i], c, sc_b[j], sc_a[i]);
        } else {
            acc[i][j] = Op::mma(fb[buf][j], fa[buf][i], c);
        }
    };
    auto read_one = [&](int buf, const char* st, int s, int x) {
        if (x < FM)
            fa[buf][x] = frag_a(st, x, s);
        else
            fb[buf][x - FM] = frag_b(st, x - FM, s);
    };
    // Register-staged copies: stg[x] holds copy x of the slice being written
    // (the copy stream's slice fg); `fc`/`foff` run one slice ahead, on the
    // slice whose loads refill stg.  Lane l of copy x writes the same LDS
    // bytes as the DMA form would.
    // NVFP4: stg[2x + h] holds half h (32 elements) of task x's row.  WIDE:
    // stg[4x + 2p + h] holds half h of slice p of a pair of slices, all four
    // loaded together at the pair's first slice (its 64 bytes are one fetch
    // of the row's cache line instead of two), and stq[x] is the slice's
    // place in its group of four.  The scales stay in their loaded form up
    // to their use (a widening or a merge right after the load would wait
    // for it): two bytes per half, or (WIDE) the 16 bytes of four slices.
    constexpr bool NV4W = nv4_wide<Op>();
    i32x4_t stg[VG ? (NV4 ? (NV4W ? 4 : 2) * LOADS : LOADS) : 1];
    uint16_t stsc[NV4 && !NV4W ? 2 * LOADS : 1];
    i32x4_t stsw[NV4W ? LOADS : 1];
    int stq[NV4W ? LOADS : 1];
    // WIDE: parity of the slice the copies now being issued write (their
    // loads fetch the next slice, so a pair is fetched when this is 1).  The
    // slice loop sets it before each step that carries copies; unrolled by
    // two, it is a constant there and the copies carry no branch.
    int nv_wpar = 0;
    // Lane l takes row 16 (l / 16) + 2 (l % 8) + (l / 8) % 2 of its wave's 64:
    // each 8-lane group of a 16-byte LDS write then holds 8 rows of one
    // parity whose swizzles (r / 2) % 8 all differ, so the group's 128 bytes
    // fall in distinct banks (consecutive rows would pair up on each bank).
    const int nv_rho = 16 * (lane >> 4) + 2 * (lane & 7) + ((lane >> 3) & 1);
    auto nv_task = [&](int x, bool& in_a, int& r) {
        const int tw = kWaveSize * wave + kThreads * x;  // wave-uniform
        in_a = tw < BM;
        r = tw + nv_rho - (in_a ? 0 : BM);
    };
    auto load_one = [&](int x) {
        if constexpr (NV4) {
            bool in_a;
            int r;
            nv_task(x, in_a, r);
            const uint32_t eoff = (uint32_t)r * (K / 2) + nv_k0 / 2;
            const uint32_t soff = (uint32_t)r * (K / 16) + nv_k0 / 16;
            if constexpr (NV4W) {
                // K % 256 == 0: a pair of slices and a group of four are
                // whole.  nv_k0 = -1 past the last slice gives place 3:
                // nothing loaded.
                stq[x] = (nv_k0 >> 6) & 3;
                if (nv_wpar == 1) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        stg[4 * x + c] = __builtin_bit_cast(
                            i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(in_a ? ra : rb, eoff + 16 * c, 0, 0));
                }
                if (stq[x] == 0)
                    stsw[x] = __builtin_bit_cast(
                        i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(in_a ? rsa : rsb, soff, 0, 0));
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bool ok = nv_k0 >= 0 && nv_k0 + 32 * h < K;
                    stg[2 * x + h] = __builtin_bit_cast(
                        i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(in_a ? ra : rb,
                                                                       ok ? eoff + 16 * h : kOutOfRange, 0, 0));
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bool ok = nv_k0 >= 0 && nv_k0 + 32 * h < K;
                    stsc[2 * x + h] = __builtin_amdgcn_raw_buffer_load_b16(
                        in_a ? rsa : rsb, ok ? soff + 2 * h : kOutOfRange, 0, 0);
                }
            }
        } else if constexpr (VG) {
            const __amdgpu_buffer_rsrc_t r = x < A_LOADS ? ra : rb;
            const uint32_t off = x < A_LOADS ? foff_a(x) : foff_b(x - A_LOADS);
            stg[x] = __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        }
    };
    // Register-staged copy x into stage st.  NVFP4: dword j of half h holds
    // elements 8j .. 8j+7 of the half (element 2i in the low nibble of byte
    // i); each byte converts to two fp16 values (v_cvt_scalef32_pk_f16_fp4
    // with scale 1; its scale operand takes only a power of two) and is
    // multiplied by its block's scale in fp16, exactly: logical fp16 chunk
    // 4 h + j of row r.  The row's scale bytes of the slice: byte 2h + b
    // scales elements 16b .. 16b+15 of half h.
    auto write_one = [&](int st, int x) {
        char* sa = lds + st * STAGE;
        if constexpr (NV4) {
            bool in_a;
            int r;
            nv_task(x, in_a, r);
            char* row = sa + (in_a ? 0 : A_BYTES) + r * RB;
            const int xs = (r >> SWZ) & (CPR - 1);
            uint32_t sw = 0;
            if constexpr (NV4W) {
                const int q = stq[x];
                const i32x4_t v = stsw[x];
                sw = (uint32_t)(q == 0 ? v[0] : q == 1 ? v[1] : q == 2 ? v[2] : v[3]);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                _Float16 s0, s1;
                if constexpr (NV4W) {
                    s0 = (_Float16)(h == 0 ? __builtin_amdgcn_cvt_f32_fp8(sw, 0)
                                           : __builtin_amdgcn_cvt_f32_fp8(sw, 2));
                    s1 = (_Float16)(h == 0 ? __builtin_amdgcn_cvt_f32_fp8(sw, 1)
                                           : __builtin_amdgcn_cvt_f32_fp8(sw, 3));
                } else {
                    s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((uint32_t)stsc[2 * x + h], 0);
                    s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((uint32_t)stsc[2 * x + h], 1);
                }
                // (both candidates read as values first: a choice between two
                // array elements would become a load from a chosen address,
                // which keeps the array out of registers)
                i32x4_t src;
                if constexpr (NV4W) {
                    const i32x4_t first = stg[4 * x + h], second = stg[4 * x + 2 + h];
                    src = nv_wpar ? second : first;
                } else {
                    src = stg[2 * x + h];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w = (uint32_t)src[j];
                    const f16x2_t s = j < 2 ? (f16x2_t){s0, s0} : (f16x2_t){s1, s1};
                    const f16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
                    const f16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
                    const f16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
                    const f16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
                    const i32x4_t chunk = {__builtin_bit_cast(int, v0), __builtin_bit_cast(int, v1),
                                           __builtin_bit_cast(int, v2), __builtin_bit_cast(int, v3)};
                    *(i32x4_t*)(row + ((4 * h + j) ^ xs) * 16) = chunk;
                }
            }
        } else {
            char* dst = x < A_LOADS ? sa + (4 * x + wave) * 1024
                                    : sa + A_BYTES + (4 * (x - A_LOADS) + wave) * 1024;
            *(i32x4_t*)(dst + lane * 16) = stg[x];
        }
    };
    auto copy_one = [&](int st, int x) {
        char* sa = lds + st * STAGE;
        if constexpr (VG) {
            write_one(st, x);
            load_one(x);
        } else if (x < A_LOADS) {
            dma(ra, sa + (4 * x + wave) * 1024, foff_a(x));
        } else {
            dma(rb, sa + A_BYTES + (4 * (x - A_LOADS) + wave) * 1024, foff_b(x - A_LOADS));
        }
    };

    // Epilogue of the C-input kernels, with a per-element operation: the wave's
    // fp32 accumulators go, OPJ 32-column blocks at a time (all 32 rows, so
    // every lane writes), to a wave-private LDS area in the MFMA layout, and
    // are read back as 16-byte row pieces (4 consecutive columns per lane,
    // whole rows per group of lanes).  Each lane then combines
    // alpha * sum + beta * c, applies the operation and stores, so C is read
    // and Out written row by row.  The loop over passes is not unrolled and
    // the read-back body exists once per operation: an operation unrolled
    // over all 256 accumulators of a lane does not fit the registers.  Every
    // element is read before it is written, by one lane, so C may be Out.
    auto op_epilogue = [&](const TileCursor& c) {
        if constexpr (AB && OPJ > 0) {
            constexpr int ROWB = OPJ * 32 * 4;           // bytes of one staged row
            constexpr int CHK = ROWB / 16;               // 16-byte chunks per row
            constexpr int RPI = kWaveSize / CHK;         // rows per read-back instruction
            constexpr int ITER = 32 / RPI;               // read-back instructions per pass
            constexpr int BATCH = ITER < 8 ? ITER : 8;   // pieces in flight at once
            constexpr int JP = FN / OPJ;                 // passes per 32-row block
            // chunk swizzle: 16 consecutive lanes of a write (16 rows, one
            // chunk) or of a read (whole rows) cover the 64 banks
            auto swz = [](int r) { return CHK >= 16 ? (r & 15) : ((r >> 1) & (CHK - 1)); };
            char* stg = lds + S * STAGE + wave * OP_BYTES;
            char* Cb = (char*)p.C + c.batch * p.stride_c;
            const char* Cinb = (const char*)p.Cin + c.batch * p.stride_cin;
            const int ldc = p.ldc;
            const bool vec = (ldc & 3) == 0;
            const bool vec_c = (p.ldcin & 3) == 0;
            const bool use_c = p.beta != 0.0f;
            const int cdt = p.c_dtype;
            const int ces = cdt == 2 ? 4 : 2;
            const float al = p.alpha, be = p.beta;
            const int row0 = c.tm * BM + wm * WTM;   // the wave's first output row
            const int col0 = c.tn * BN + wn * WTN;
            // pass P: rows of block i = P / JP, column blocks (P % JP) OPJ + 0..OPJ-1
            auto stage = [&](auto P) {
                constexpr int i = decltype(P)::value / JP, jg = decltype(P)::value % JP;
#pragma unroll
                for (int jj = 0; jj < OPJ; ++jj)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x16_t& a = acc[i][jg * OPJ + jj];
                        const int ch = (8 * jj + 2 * q + hi) ^ swz(l32);
                        lds_write16_acc(stg + l32 * ROWB + ch * 16,
                                        (f32x4_t){a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]});
                    }
            };
            auto readback = [&](auto OPC, int m0, int n0) {
                constexpr int OP = decltype(OPC)::value;
                const int ck = lane % CHK;
                const int n = n0 + 4 * ck;
                const bool vec4 = vec && n + 3 < p.N;
#pragma unroll
                for (int t0 = 0; t0 < ITER; t0 += BATCH) {
                    // the batch's row pieces and their C values in flight first,
                    // then one scheduling region per piece
                    f32x4_t a4[BATCH], c4[BATCH];
#pragma unroll
                    for (int t = 0; t < BATCH; ++t) {
                        const int r = (t0 + t) * RPI + lane / CHK;
                        a4[t] = *(const f32x4_t*)(stg + r * ROWB + ((ck ^ swz(r)) * 16));
                    }
#pragma unroll
                    for (int t = 0; t < BATCH; ++t) {
                        const int m = m0 + (t0 + t) * RPI + lane / CHK;
                        c4[t] = (f32x4_t){};
                        if (use_c && m < p.M) {
                            const char* crow = Cinb + (int64_t)m * p.ldcin * ces;
                            if (vec_c && vec4) {
                                c4[t] = load4_c(crow, n, cdt);
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (n + e < p.N) c4[t][e] = load1_c(crow, n + e, cdt);
                            }
                        }
                    }
#pragma unroll
                    for (int t = 0; t < BATCH; ++t) {
                        __builtin_amdgcn_sched_barrier(0);
                        const int m = m0 + (t0 + t) * RPI + lane / CHK;
                        if (m >= p.M) continue;
                        TOut* orow = (TOut*)Cb + (int64_t)m * ldc;
                        f32x4_t v = {al * a4[t][0], al * a4[t][1], al * a4[t][2], al * a4[t][3]};
                        if (use_c) v += be * c4[t];
                        if (vec4) {
                            store4<TOut>(orow + n, apply_op<OP>(v[0]), apply_op<OP>(v[1]),
                                         apply_op<OP>(v[2]), apply_op<OP>(v[3]));
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (n + e < p.N)
                                    orow[n + e] = convert_out<TOut>(apply_op<OP>(v[e]));
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
#pragma unroll 1
            for (int pass = 0; pass < FM * JP; ++pass) {
                static_for<FM * JP>([&](auto P) {
                    if (pass == decltype(P)::value) stage(P);
                });
                // the wave's own LDS writes, then reads by other lanes
                wave_lds_exchange();
                const int m0 = row0 + (pass / JP) * 32;
                const int n0 = col0 + (pass % JP) * OPJ * 32;
                switch (p.op) {
                case kOpIdentity: readback(std::integral_constant<int, kOpIdentity>{}, m0, n0); break;
                case kOpRelu: readback(std::integral_constant<int, kOpRelu>{}, m0, n0); break;
                case kOpGeluTanh: readback(std::integral_constant<int, kOpGeluTanh>{}, m0, n0); break;
                case kOpGeluErf: readback(std::integral_constant<int, kOpGeluErf>{}, m0, n0); break;
                default: readback(std::integral_constant<int, kOpSilu>{}, m0, n0);
                }
                wave_lds_exchange();
            }
        }
    };

    auto epilogue = [&](const TileCursor& c) {
        // Out's row stride, read from the arguments here (a value held from
        // the kernel's start costs the main loop a register)
        const int ldc = DENSE ? p.N : p.ldc;
        char* Cb = (char*)p.C + c.batch * p.stride_c;
        const int m_base = c.tm * BM + wm * WTM + l32;
        const int n_base = c.tn * BN + wn * WTN + 4 * hi;
        const bool full = c.tm * BM + BM <= p.M && c.tn * BN + BN <= p.N && (ldc & 3) == 0;
        if constexpr (AB && OPJ > 0) {
            // an interior tile of a product without C or operation takes the
            // 16-bit staged form below (alpha applied there) where the kernel
            // has it; every other tile keeps the alpha/beta epilogue
            if (!(EPI_LDS && p.beta == 0.0f && p.op == 0 && full &&
                  ldc % (16 / (int)sizeof(TOut)) == 0)) {
                op_epilogue(c);
                return;
            }
        } else if constexpr (AB) {
            // (tiles without room for the staged form: no operation)
            // Each lane reads the C values of exactly the outputs it writes,
            // so C may be the output itself (an in-place update).
            const bool vec = (ldc & 3) == 0;
            const bool vec_c = (p.ldcin & 3) == 0;
            const bool use_c = p.beta != 0.0f;
            const int cdt = p.c_dtype;
            const int ces = cdt == 2 ? 4 : 2;
            const char* Cinb = (const char*)p.Cin + c.batch * p.stride_cin;
            const float al = p.alpha, be = p.beta;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = m_base + i * 32;
                if (m >= p.M) continue;
                TOut* row = (TOut*)Cb + (int64_t)m * ldc;
                const char* crow = Cinb + (int64_t)m * p.ldcin * ces;
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = n_base + j * 32 + 8 * q;
                        const f32x16_t& a4 = acc[i][j];
                        if (vec && n + 3 < p.N) {
                            f32x4_t v = {al * a4[4 * q], al * a4[4 * q + 1], al * a4[4 * q + 2],
                                         al * a4[4 * q + 3]};
                            if (use_c)
                                v += be * (vec_c ? load4_c(crow, n, cdt)
                                                 : (f32x4_t){load1_c(crow, n, cdt),
                                                             load1_c(crow, n + 1, cdt),
                                                             load1_c(crow, n + 2, cdt),
                                                             load1_c(crow, n + 3, cdt)});
                            store4<TOut>(row + n, v[0], v[1], v[2], v[3]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (n + e < p.N) {
                                    float x = al * a4[4 * q + e];
                                    if (use_c) x += be * load1_c(crow, n + e, cdt);
                                    row[n + e] = convert_out<TOut>(x);
                                }
                        }
                    }
            }
            return;
        }
        if constexpr (EPI_LDS) {
            // Interior tiles go through LDS: each 32-row block of the wave's
            // output is written to the wave's staging area in the MFMA layout,
            // read back as 16-byte row pieces, and stored so that every store
            // instruction writes whole 256-byte row segments (4 rows for
            // bf16, 2 for fp32) instead of 16-byte pieces of 32 rows.
            if (full && ldc % (16 / (int)sizeof(TOut)) == 0) {
                constexpr int CHK = STG_ROWB / 16;          // 16-byte chunks per staged row
                constexpr int RPI = kWaveSize * 16 / STG_ROWB;  // rows per store instruction
                char* stg = lds + S * STAGE + wave * STG_BYTES;
                // The lane index is taken afresh here: the per-lane LDS and
                // row offsets below would otherwise be computed once before
                // the tile loop and kept in registers across the K loop,
                // which has none to spare (they were spilled, and each
                // reload's wait also waited for the stores before it).
                const int lane = (int)__builtin_amdgcn_mbcnt_hi(
                    ~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
                const int row_l = lane & 31;                 // staged row this lane writes
                const int hi = lane >> 5;
                // alpha of the C-input kernels (1 elsewhere: the product alone)
                const float al = AB ? p.alpha : 1.0f;
#pragma unroll
                for (int i = 0; i < FM; ++i) {
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const f32x16_t& a4 = acc[i][j];
                            const int col = j * 32 + 8 * q + 4 * hi;  // column within the wave tile
                            const int byte = col * (int)sizeof(TOut);
                            const int chunk = (byte / 16) ^ (row_l & (CHK - 1));
                            char* dst = stg + row_l * STG_ROWB + chunk * 16 + byte % 16;
                            store4<TOut>((TOut*)dst, al * a4[4 * q], al * a4[4 * q + 1],
                                         al * a4[4 * q + 2], al * a4[4 * q + 3]);
                        }
                    // same-wave LDS writes then reads: the wave's own order holds
                    wave_lds_exchange();
#pragma unroll
                    for (int t = 0; t < 32 / RPI; ++t) {
                        const int r = t * RPI + lane / CHK;
                        const int ck = lane % CHK;
                        const i32x4_t d = *(const i32x4_t*)(stg + r * STG_ROWB +
                                                            ((ck ^ (r & (CHK - 1))) * 16));
                        char* g = Cb + ((int64_t)(c.tm * BM + wm * WTM + i * 32 + r) * ldc +
                                        c.tn * BN + wn * WTN) * (int64_t)sizeof(TOut) + ck * 16;
                        *(i32x4_t*)g = d;
                    }
                    wave_lds_exchange();
                }
                return;
            }
        }
        if (full) {
            // interior tile: one 4-wide store per (block, r / 4), no masks
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                TOut* row = (TOut*)Cb + (int64_t)(m_base + i * 32) * ldc + n_base;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        store4<TOut>(row + j * 32 + 8 * q, acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                     acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            // edge tile: rows past M and columns past N are not written
            const bool vec = (ldc & 3) == 0;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = m_base + i * 32;
                if (m >= p.M) continue;
                TOut* row = (TOut*)Cb + (int64_t)m * ldc;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = n_base + j * 32 + 8 * q;
                        if (vec && n + 3 < p.N) {
                            store4<TOut>(row + n, acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                         acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (n + e < p.N) row[n + e] = convert_out<TOut>(acc[i][j][4 * q + e]);
                        }
                    }
                }
            }
        }
    };

    // ---- schedule of one K step ---------------------------------------------
    // The issue order inside a K step is pinned: MFMA x, then copy x (when the
    // step carries copies), then fragment read x, with a scheduling barrier
    // after each triple.  Each MFMA occupies the matrix core for many cycles,
    // so the reads and copies of a triple issue in its shadow and the next
    // MFMA is ready when the matrix core frees up.
    constexpr int N_MFMA = FM * FN;
    constexpr int N_FRAG = FM + FN;
    // `nc` copies ride in the step (at most PMAX; a constant once the K-step
    // loop is unrolled).
    auto kstep = [&](int buf, int s, const char* rd_st, int rd_s, int copy_st, int copy_base,
                     int nc, auto ZERO) {
        constexpr int NM = N_MFMA > N_FRAG ? N_MFMA : N_FRAG;
        constexpr int NX = NM > PMAX ? NM : PMAX;
        // Copies go out after every second MFMA where the step has room for
        // that (fewer back-to-back copies in the address FIFOs; measured
        // better than back-to-back and than every fourth), the reads of the
        // next step's fragments after the first MFMAs.
        constexpr int CS = 2 * PMAX <= N_MFMA ? 2 : 1;
#pragma unroll
        for (int x = 0; x < NX; ++x) {
            if (x < N_MFMA) mma_one(buf, s, x, ZERO);
            if (x % CS == 0 && x / CS < nc) copy_one(copy_st, copy_base + x / CS);
            if (x < N_FRAG) read_one(buf ^ 1, rd_st, rd_s, x);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- the copy stream's schedule -----------------------------------------
    // The copies of slice g + S go out in NSPLIT parts: part 0 in slice g's
    // hand-off step (right after the barrier frees stage g % S), parts
    // 1 .. NSPLIT-1 in the first K steps of slice g + 1.  Spreading them keeps
    // the per-CU request rate within what the vector L1 can pass to L2; a
    // burst of a whole stage fills the address FIFOs and stalls MFMA issue.
    int fg = 0;  // global slice index of the copy stream
    auto feed_next = [&]() {
        feed_advance();
        ++fg;
        feed_offsets(fg + (VG ? 1 : 0) < total);
    };

    // ---- prologue: slices 0 .. S-2 and part 0 of slice S-1 in flight -------
    locate(fc);
    feed_resources();
    TileCursor cc = fc;
    feed_offsets(true);
    if constexpr (VG) {
        // slice 0 straight into stage 0; slice 1 into registers, the load
        // stream moved on to slice 2, and part 0 of slice 1 written
        nv_wpar = 1;  // (the loads of slice 0 start a pair)
#pragma unroll
        for (int x = 0; x < LOADS; ++x) load_one(x);
        nv_wpar = 0;
#pragma unroll
        for (int x = 0; x < LOADS; ++x) write_one(0, x);
        feed_advance();
        feed_offsets(1 < total);
#pragma unroll
        for (int x = 0; x < LOADS; ++x) load_one(x);  // slice 1: nothing for WIDE (nv_wpar 0)
        feed_advance();
        fg = 1;
        feed_offsets(2 < total);
        nv_wpar = 1;
#pragma unroll
        for (int x = 0; x < PART; ++x) copy_one(1, x);
        if constexpr (NSPLIT == 1) feed_next();
        barrier_lds();
    } else {
#pragma unroll
        for (int g = 0; g < S - 1; ++g) {
            issue(g);
            feed_next();
        }
#pragma unroll
        for (int x = 0; x < PART; ++x) copy_one(S - 1, x);
        if constexpr (NSPLIT == 1) feed_next();
        wait_vmcnt<(S - 2) * LOADS + PART>();
        barrier_lds();
    }
    read_frags(0, lds, 0);
    if constexpr (Op::kScaled) load_scales(cc, sc_a, sc_b);

    // One slice g: K steps with double-buffered fragments.  The stage
    // hand-off sits before the last K step: once this wave's copies of slice
    // g + 1 have landed and every wave has passed the barrier, stage g % S is
    // free for the copies of slice g + S, and the first fragments of slice
    // g + 1 are read while the last K step's MFMAs run.  ZERO marks a tile's
    // first slice, whose first MFMAs take a zero accumulator.
    bool after_epilogue = false;
    // PAR: g's parity as a constant (0 or 1), or -1 where it is not fixed.
    auto slice = [&](int g, auto ZERO, auto PAR) {
        constexpr int par = decltype(PAR)::value;
        const char* st = lds + (g % S) * STAGE;
        const char* st_next = lds + ((g + 1) % S) * STAGE;
        if constexpr (Op::kScaled) {
            TileCursor nc = cc;
            advance(nc);
            if (g + 1 < total) load_scales(nc, nx_a, nx_b);
        }
        __builtin_amdgcn_sched_barrier(0);
        constexpr int NONE = 0;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const int cur = s & 1;
            const bool zero = decltype(ZERO)::value && s == 0;
            if (s + 1 < KSTEPS) {
                if (s + 1 < NSPLIT) {
                    // a later part of slice g - 1 + S, into stage (g - 1) % S
                    const int cst = (g + S - 1) % S;
                    nv_wpar = par >= 0 ? (par + S - 1) & 1 : (g + S - 1) & 1;
                    if (zero)
                        kstep(cur, s, st, s + 1, cst, part_base(s + 1),
                              part_base(s + 2) - part_base(s + 1), std::true_type{});
                    else
                        kstep(cur, s, st, s + 1, cst, part_base(s + 1),
                              part_base(s + 2) - part_base(s + 1), std::false_type{});
                    if (s + 2 == NSPLIT) feed_next();
                } else {
                    if (zero)
                        kstep(cur, s, st, s + 1, 0, 0, NONE, std::true_type{});
                    else
                        kstep(cur, s, st, s + 1, 0, 0, NONE, std::false_type{});
                }
            } else {
                // register-staged copies: their writes are LDS operations,
                // covered by the barrier's lgkmcnt wait
                if constexpr (VG) {
                } else if (S > 2 && !after_epilogue && g + S - 1 < total) {
                    wait_vmcnt<(S > 2 ? (S - 2) * LOADS : 0)>();
                } else {
                    wait_vmcnt<0>();
                }
                after_epilogue = false;
                barrier_lds();
                __builtin_amdgcn_sched_barrier(0);
                nv_wpar = par >= 0 ? (par + S) & 1 : (g + S) & 1;  // part 0 of slice g + S
                if (zero)
                    kstep(cur, s, st_next, 0, g % S, 0, PART, std::true_type{});
                else
                    kstep(cur, s, st_next, 0, g % S, 0, PART, std::false_type{});
            }
        }
        if constexpr (NSPLIT == 1) feed_next();
    };

    int g = 0;
    using P_ANY = std::integral_constant<int, -1>;
    using P_EVEN = std::integral_constant<int, 0>;
    using P_ODD = std::integral_constant<int, 1>;
    for (int tl = 0; tl < my_tiles; ++tl) {
        if constexpr (NV4W) {
            // slices in pairs (a tile's slice count is a multiple of 4 here,
            // and g counts from 0): first, (odd, even) pairs, last
            slice(g, std::true_type{}, P_EVEN{});
            ++g;
            for (int kk = 1; kk + 1 < p.ksteps; kk += 2, g += 2) {
                slice(g, std::false_type{}, P_ODD{});
                slice(g + 1, std::false_type{}, P_EVEN{});
            }
            slice(g, std::false_type{}, P_ODD{});
            ++g;
            TileCursor ec = {tl, 0, 0, 0, 0};
            locate(ec);
            __builtin_amdgcn_sched_barrier(0);
            epilogue(ec);
            __builtin_amdgcn_sched_barrier(0);
            after_epilogue = true;
            continue;
        }
        slice(g, std::true_type{}, P_ANY{});
        if constexpr (Op::kScaled) {
            advance(cc);
#pragma unroll
            for (int i = 0; i < FM; ++i) sc_a[i] = nx_a[i];
#pragma unroll
            for (int j = 0; j < FN; ++j) sc_b[j] = nx_b[j];
        }
        ++g;
        for (int kk = 1; kk < p.ksteps; ++kk, ++g) {
            slice(g, std::false_type{}, P_ANY{});
            if constexpr (Op::kScaled) {
                advance(cc);
#pragma unroll
                for (int i = 0; i < FM; ++i) sc_a[i] = nx_a[i];
#pragma unroll
                for (int j = 0; j < FN; ++j) sc_b[j] = nx_b[j];
            }
        }
        // Epilogue of this tile, while the copies of the next tile's first
        // slices and the reads of its first fragments are in flight.
        TileCursor ec = {tl, 0, 0, 0, 0};
        locate(ec);
        __builtin_amdgcn_sched_barrier(0);
        epilogue(ec);
        __builtin_amdgcn_sched_barrier(0);
        after_epilogue = true;
    }
}

}  // namespace tcm
