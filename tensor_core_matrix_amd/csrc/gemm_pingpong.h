// Ping-pong variant of the tiled product kernel for gfx950: a 256 x 256
// output tile, eight waves, two per SIMD, taking turns on the matrix core.
//
// "Hopper and Blackwell GEMM" (Concept) describes two consumer warpgroups
// taking turns so that one group's epilogue hides under the other's MMAs,
// and a producer that only issues loads.  On CDNA4 every wave of a kernel
// gets the same register budget, so a producer-only wave cannot sit beside
// waves holding a large accumulator.  Here the roles alternate within each
// wave instead:
//
//  * Group 0 (waves 0-3) owns output rows 0-127 of the tile, group 1 (waves
//    4-7) rows 128-255; wave w of a group owns columns 64 (w % 4) .. +63.
//    Each wave holds a 128 x 64 fp32 accumulator (128 registers) and the
//    fragments of one K unit.
//  * K is walked in units of UNIT_K.  Time is cut into half-periods separated
//    by workgroup barriers: in half 2u group 0 runs the MFMAs of unit u while
//    group 1 reads its fragments of unit u from LDS; in half 2u+1 group 1 runs
//    unit u while group 0 reads unit u+1.  A wave in its MFMA half issues
//    nothing but MFMAs, so the stalls of reads and copies (LDS latency, full
//    address FIFOs) fall on the other wave and the matrix core of each SIMD
//    stays busy.
//  * An S-stage LDS ring of units (S >= 3).  Unit v is read in halves 2v-1
//    and 2v, so its stage is free from half 2v+1 on; the copies of unit v+S
//    into it are issued in the memory halves of unit v+1, shared by both
//    groups, and waited for by their issuing waves just before the barrier
//    that precedes the first read of unit v+S.  With S = 4 a copy has four
//    half-periods to land and each memory half issues a quarter of what a
//    two-stage ring would need in one.  (A two-stage ring, with group 0
//    alone copying because group 1's share would have to land within the
//    half it is issued in, measured far slower.)
//  * The epilogue of a tile runs in each wave's memory half right after its
//    last MFMA half -- while the other group computes -- staged through a
//    wave-private LDS area so that every store writes whole row segments.
//    This is the two-accumulator overlap of the pages, the second
//    accumulator set being the other group's.
#pragma once

#include <type_traits>

#include "gemm_kernel.h"

namespace tcm {

constexpr int kPPThreads = 512;  // eight waves

// SCALE_MODE (MX only) says how the E8M0 rows may be read: 0 byte by byte,
// 1 as 32-bit words (K a multiple of 128, word-aligned arrays), 2 as 16-byte
// pieces (K a multiple of 512, 16-byte-aligned arrays).
// A_MN (B_MN): MXFP8 A stored M-major (B N-major), K rows of lda (ldb)
// bytes; the stage then holds the unit's 64 k rows of the tile's 256 values,
// read with ds_read_b64_tr_b8 as in the 4-wave kernel, and the K-major
// operand's rows are lda (ldb) bytes apart.  Every DMA is then issued as
// inline assembly (see copy16_to_lds_asm).
template <class Op, typename TOut, int UNIT_K, int S, int SCALE_MODE = 0, bool A_MN = false,
          bool B_MN = false>
__global__ __launch_bounds__(kPPThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void pingpong_gemm_kernel(GemmArgs p) {
    constexpr int BM = 256, BN = 256;
    constexpr int EBITS = Op::kElemBits;
    constexpr bool FP6 = EBITS == 6;
    constexpr int BK = UNIT_K;
    constexpr int RB = BK * EBITS / 8;  // bytes of one operand row's K unit
    constexpr int CPR = RB / 16;        // 16-byte chunks per row
    // FP6 rows of a 64-deep unit are 48 bytes (CPR = 3 chunks), stored row
    // after row without a swizzle: chunk k of row r is chunk 3 r + k of the
    // operand region.  16 lanes reading one chunk of 16 consecutive rows
    // touch chunks 3 r + k, which fall on 16 different 16-byte bank groups
    // (3 r mod 16 takes every value once over 16 rows).  A copy's
    // consecutive lanes take consecutive chunks, so each row's 48 bytes are
    // fetched by three neighbouring lanes from one contiguous stretch of
    // memory (a lane per row, as in a chunk-major layout, made the vector L1
    // look up a separate cache line for nearly every lane).
    // chunk ^= row bits chosen so that the 16 rows read together by 16 lanes
    // fall on 16 different 16-byte bank groups (64 banks of 4 bytes)
    constexpr int SWZ = CPR == 8 ? 1 : 2;
    // FP6 with 128-deep units (PAIR6): rows of 96 bytes (6 chunks), chunk k
    // of row r at chunk 6 r + (k ^ ((r >> 3) & 1)).  Over 16 consecutive
    // rows 6 r mod 16 takes each even value twice, for rows r and r + 8; the
    // XOR moves rows 8-15 of every 16 to the odd bank groups, so 16 lanes
    // reading chunk k of 16 consecutive rows meet no conflict.  The MFMA's
    // two K blocks per lane half are blocks {0, 2} (first K step) and {1, 3}
    // (second) of the unit's four: then both lane halves start their
    // 24-byte operand at a chunk boundary (bytes 0 and 48, then 24 and 72),
    // and three 16-byte reads give both K steps' operands with no byte read
    // twice (see read_pair6).
    constexpr bool PAIR6 = FP6 && BK == 128;
    constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB, DATA = A_BYTES + B_BYTES;
    // MX scales reach the MFMA waves through LDS, copied by the same DMA as
    // the operands, so that no wave waits on a global load.  With 16-byte
    // pieces (SC_CHUNK) one DMA per wave brings 16 blocks of 64 rows, the
    // scales of UPC units, into one of two chunk buffers after the ring;
    // with 32-bit words (SC_LDS) every stage ends with one word per A and B
    // row, the 4 blocks that hold the unit's blocks.  A DMA lane touches one
    // row, so fewer, wider pieces keep the address unit free for operands.
    constexpr bool SCALE_WORDS = SCALE_MODE >= 1;
    constexpr bool SC_CHUNK = Op::kScaled && SCALE_MODE == 2;
    constexpr bool SC_LDS = Op::kScaled && SCALE_MODE == 1;
    constexpr int SC_BYTES = SC_LDS ? (BM + BN) * 4 : 0;
    constexpr int STAGE = DATA + SC_BYTES;
    constexpr int UPC = 16 / (BK / 32);                       // units per scale chunk
    constexpr int CHUNK_BYTES = (BM + BN) * 16;
    constexpr int SC_CHUNK_TOTAL = SC_CHUNK ? 2 * CHUNK_BYTES : 0;
    constexpr int WTM = 128, WTN = 64, FM = WTM / 32, FN = WTN / 32;
    constexpr int KSTEPS = BK / Op::kK;
    constexpr int CPL = Op::kK * EBITS / 8 / 32;  // 16-byte chunks per lane per MFMA (>= 8 bits)
    // copies: 1 KiB per wave instruction, shared by all eight waves
    constexpr int NCW = 8;                             // copying waves
    constexpr int A_COPIES = A_BYTES / 1024;
    constexpr int PW = DATA / 1024 / NCW;              // operand copies per wave per unit
    constexpr int OPS = PW + (SC_LDS ? 1 : 0);         // DMA operations per wave per unit
    constexpr int RPC = FP6 ? 16 : 1024 / RB;          // rows per copy instruction (not FP6)
    // epilogue staging: 32 (or, where the ring leaves less room, 16) rows x
    // 64 columns per wave (bf16 only, and only where 16 rows fit)
    constexpr int STG_ROWB = WTN * (int)sizeof(TOut);
    constexpr int RING = S * STAGE + SC_CHUNK_TOTAL;
    constexpr bool EPI_LDS = sizeof(TOut) == 2 && RING + 8 * 16 * STG_ROWB <= 160 * 1024;
    constexpr int STG_ROWS = RING + 8 * 32 * STG_ROWB <= 160 * 1024 ? 32 : 16;
    constexpr int STG_BYTES = EPI_LDS ? STG_ROWS * STG_ROWB : 0;
    static_assert(CPR == 4 || CPR == 8 || (FP6 && (BK == 64 || BK == 128)),
                  "64- or 128-byte rows, or FP6 units 64 or 128 deep (48- or 96-byte rows)");
    static_assert(KSTEPS >= 1 && KSTEPS <= 4, "K steps per unit");
    static_assert(!Op::kScaled || KSTEPS <= 2, "scale bytes per register");
    static_assert((DATA / 1024) % NCW == 0, "copy split");
    static_assert(STAGE % 1024 == 0, "stage alignment");
    static_assert(RING + 8 * STG_BYTES <= 160 * 1024, "LDS budget");
    static_assert(S * OPS < 64, "vmcnt range");
    static_assert(S >= 3, "ring of at least three units");
    static_assert(!SC_CHUNK || UPC * KSTEPS == 8, "8 packed scale bytes per lane per chunk");
    static_assert(!SC_CHUNK || UPC >= 2, "a chunk lands two halves after its DMA");
    static_assert(FP6 || (32 >> SWZ) % CPR == 0, "swizzle depends on the row within 32 only");
    constexpr bool ANY_MN = A_MN || B_MN;
    static_assert(!ANY_MN || (EBITS == 8 && Op::kScaled && BK == 64),
                  "M/N-major operands: MXFP8, 64-deep units");

    __shared__ __attribute__((aligned(1024))) char lds[RING + 8 * STG_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, sub = wave & 3;
    const int l32 = lane & 31, hi = lane >> 5;

    const int G = gridDim.x;
    const int lid = logical_block(blockIdx.x, G);
    if (lid >= p.total_tiles) return;
    const int my_tiles = (p.total_tiles - 1 - lid) / G + 1;
    const int T = my_tiles * p.ksteps;  // K units of this workgroup
    const int K = p.K;
    const uint32_t ROWB = (uint32_t)K * EBITS / 8;  // bytes of a whole operand row
    // row strides of the stored operands: whole rows (K-major, dense) or the
    // leading dimensions (kernels with an M/N-major operand)
    const uint32_t ROWB_A = ANY_MN ? (uint32_t)p.lda : ROWB;
    const uint32_t ROWB_B = ANY_MN ? (uint32_t)p.ldb : ROWB;

    auto locate = [&](TileCursor& c) { tile_coords(p, c.tl * G + lid, c.batch, c.tm, c.tn); };
    auto advance = [&](TileCursor& c) {
        if (++c.kk == p.ksteps) {
            c.kk = 0;
            if (++c.tl < my_tiles) locate(c);
        }
    };

    // ---- copy stream: this wave's share of every unit --------------------------
    // Copy t of this wave is instruction q = cw + t * NCW of the unit (cw =
    // this wave's index among the copying waves): LDS bytes [1024 q, +1024)
    // of the stage, i.e. rows RPC qq .. RPC qq + RPC - 1 of A (qq = q while
    // q < A_COPIES) or of B (qq = q - A_COPIES).  The rows of one wave's
    // copies are NCW RPC apart and the swizzle repeats every CPR << SWZ rows,
    // so a lane's chunk is the same in all of them: one lane offset serves
    // every copy, and each copy adds the wave-uniform row offset RPC qq K.
    const int cw = wave;
    static_assert(FP6 || ((NCW * RPC) % (CPR << SWZ) == 0 && (A_COPIES * RPC) % (CPR << SWZ) == 0),
                  "chunk independent of the copy");
    const int cp_row = lane / CPR;
    const int sw_row = cw * RPC + cp_row;  // congruent to every copied row of the lane
    const int cp_chunk = (lane % CPR) ^ ((sw_row >> SWZ) & (CPR - 1));
    const uint32_t cp_lane_off = (uint32_t)cp_row * ROWB + cp_chunk * 16;
    const int cp_k = cp_chunk * (128 / EBITS);  // first K element of the lane's chunk
    auto copy_row_off = [&](int t) -> uint32_t {
        const int q = cw + t * NCW;
        const int qq = q < A_COPIES ? q : q - A_COPIES;
        return (uint32_t)(qq * RPC) * ROWB;
    };
    // M/N-major operand (256-byte k rows, 16 chunks): copy qq fills k rows
    // 4 qq .. 4 qq + 3; lane l writes physical chunk l % 16 of k row
    // 4 qq + l / 16, holding logical chunk (l % 16) ^ 2 (k % 8).  A wave's
    // copies all have qq of its own parity, so k % 8 = 4 (cw % 2) + l / 16
    // and one lane offset serves every copy.
    const int mn_k = 4 * (cw & 1) + lane / 16;
    const int mn_lc = (lane % 16) ^ (2 * (mn_k & 7));
    auto mn_lane_off = [&](uint32_t ld) -> uint32_t {
        return (uint32_t)(lane / 16) * ld + (uint32_t)mn_lc * 16;
    };
    auto mn_row_off = [&](int t, uint32_t ld) -> uint32_t {
        const int q = cw + t * NCW;
        const int qq = q < A_COPIES ? q : q - A_COPIES;
        return (uint32_t)(4 * qq) * ld;
    };
    // K-major operand of a kernel with an M/N-major one: rows ld apart
    const uint32_t kmaj_lane_off_a = (uint32_t)cp_row * ROWB_A + cp_chunk * 16;
    const uint32_t kmaj_lane_off_b = (uint32_t)cp_row * ROWB_B + cp_chunk * 16;
    // FP6: copy t fills chunk Qo = 64 qq + lane of its operand region (qq the
    // copy's index within A or B): row Qo / CPR, chunk Qo % CPR.  The
    // pattern has no uniform step, so each copy keeps its own lane offset
    // and chunk byte (for the K tail).
    // Where A's copies split evenly over the copying waves, copy t of A and
    // copy t + A_COPIES / NCW (of B) have the same index within their
    // operand, so NOFF offsets serve all of them.
    constexpr int NOFF = FP6 && A_COPIES % NCW == 0 ? A_COPIES / NCW : PW;
    uint32_t off6[FP6 ? NOFF : 1];
    int cb6[FP6 ? NOFF : 1];
    if constexpr (FP6) {
#pragma unroll
        for (int t = 0; t < NOFF; ++t) {
            const int q = cw + t * NCW;
            const int qq = q < A_COPIES ? q : q - A_COPIES;
            const int Qo = 64 * qq + lane;
            const int r = Qo / CPR, k = (Qo % CPR) ^ (PAIR6 ? (r >> 3) & 1 : 0);
            off6[t] = (uint32_t)r * ROWB + 16 * k;
            cb6[t] = 16 * k;
        }
    }
    TileCursor fc = {0, 0, 0, 0, 0};
    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
    const int kblocks = K / 32;
    const uint32_t sc_lane_off = (uint32_t)((wave & 3) * 64 + lane) * (uint32_t)kblocks;
    auto feed_resources = [&]() {
        const int rows_a = min(BM, p.M - fc.tm * BM);
        const int rows_b = min(BN, p.N - fc.tn * BN);
        if constexpr (ANY_MN) {
            // M/N-major: base at the tile's first column, records up to the
            // last k row's last 16-byte piece holding a valid column, so k
            // rows past K read as zeros (ld is a multiple of 16); K-major:
            // the tile's rows of ld bytes
            const char* abase = (const char*)p.A + fc.batch * p.stride_a;
            const char* bbase = (const char*)p.B + fc.batch * p.stride_b;
            auto mn_records = [&](int rows, uint32_t ld) -> uint32_t {
                return K > 0 ? (uint32_t)(K - 1) * ld + (uint32_t)((rows + 15) & ~15) : 0u;
            };
            ra = A_MN ? make_rsrc(abase + (int64_t)fc.tm * BM, mn_records(rows_a, ROWB_A))
                      : make_rsrc(abase + (int64_t)fc.tm * BM * ROWB_A, (uint32_t)rows_a * ROWB_A);
            rb = B_MN ? make_rsrc(bbase + (int64_t)fc.tn * BN, mn_records(rows_b, ROWB_B))
                      : make_rsrc(bbase + (int64_t)fc.tn * BN * ROWB_B, (uint32_t)rows_b * ROWB_B);
            if constexpr (SC_LDS) {
                const uint8_t* sab = (const uint8_t*)p.SA + (int64_t)fc.tm * BM * kblocks;
                const uint8_t* sbb = (const uint8_t*)p.SB + (int64_t)fc.tn * BN * kblocks;
                rsa = make_rsrc(sab, (uint32_t)rows_a * (uint32_t)kblocks);
                rsb = make_rsrc(sbb, (uint32_t)rows_b * (uint32_t)kblocks);
            }
            return;
        }
        const char* abase = (const char*)p.A + fc.batch * p.stride_a + (int64_t)fc.tm * BM * ROWB;
        const char* bbase = (const char*)p.B + fc.batch * p.stride_b + (int64_t)fc.tn * BN * ROWB;
        ra = make_rsrc(abase, (uint32_t)rows_a * ROWB);
        rb = make_rsrc(bbase, (uint32_t)rows_b * ROWB);
        if constexpr (SC_LDS) {
            const uint8_t* sab = (const uint8_t*)p.SA + (int64_t)fc.tm * BM * kblocks;
            const uint8_t* sbb = (const uint8_t*)p.SB + (int64_t)fc.tn * BN * kblocks;
            rsa = make_rsrc(sab, (uint32_t)rows_a * (uint32_t)kblocks);
            rsb = make_rsrc(sbb, (uint32_t)rows_b * (uint32_t)kblocks);
        }
    };
    // scale chunks: cursor on the first unit of the next chunk to copy
    TileCursor scc = {0, 0, 0, 0, 0};
    __amdgpu_buffer_rsrc_t rca, rcb;
    auto chunk_resources = [&]() {
        const int rows_a = min(BM, p.M - scc.tm * BM);
        const int rows_b = min(BN, p.N - scc.tn * BN);
        rca = make_rsrc((const uint8_t*)p.SA + (int64_t)scc.tm * BM * kblocks,
                        (uint32_t)rows_a * (uint32_t)kblocks);
        rcb = make_rsrc((const uint8_t*)p.SB + (int64_t)scc.tn * BN * kblocks,
                        (uint32_t)rows_b * (uint32_t)kblocks);
    };
    int cu = 0;  // first unit of the chunk the scale stream is on
    // wave w copies 16 blocks of A rows 64 w .. (w < 4) or of B rows 64 (w - 4) ..
    auto issue_chunk = [&]() {
        const uint32_t off = cu < T ? sc_lane_off + (uint32_t)(scc.kk * (BK / 32)) : kOutOfRange;
        char* dst = lds + S * STAGE + ((cu / UPC) & 1) * CHUNK_BYTES + wave * 1024;
        if constexpr (ANY_MN)
            copy16_to_lds_asm(wave < 4 ? rca : rcb, dst, off);
        else
            copy16_to_lds(wave < 4 ? rca : rcb, dst, off);
        cu += UPC;
        scc.kk += UPC;
        if (scc.kk >= p.ksteps) {
            scc.kk = 0;
            if (++scc.tl < my_tiles) {
                locate(scc);
                chunk_resources();
            }
        }
    };
    int fu = 0;  // unit the copy stream is on
    // This wave's copies of unit fu into its stage.  Past the last unit every
    // offset is out of range: nothing is read and a stage that is never read
    // again receives zeros.
    // Offset of this lane's piece in copy 0 of unit fu; copy t adds the
    // wave-uniform copy_row_off(t).  Out of range (>= 2^31, beyond any
    // tile's records even with a row offset added) past the last unit and
    // for pieces past K.
    auto copy_base = [&]() -> uint32_t {
        const int k0 = fc.kk * BK;
        if constexpr (FP6)  // the unit's first byte within a row (the offsets are per copy)
            return fu < T ? (uint32_t)k0 * EBITS / 8 : kOutOfRange;
        else
            return (fu < T && k0 + cp_k < K) ? cp_lane_off + (uint32_t)k0 * EBITS / 8 : kOutOfRange;
    };
    // kernels with an M/N-major operand: the unit's offsets of A's and B's
    // lane pieces (copy t adds its row offset)
    auto copy_base_op = [&](bool mn, bool is_a) -> uint32_t {
        const int k0 = fc.kk * BK;
        const uint32_t ld = is_a ? ROWB_A : ROWB_B;
        if (fu >= T) return kOutOfRange;
        if (mn) return (uint32_t)k0 * ld + mn_lane_off(ld);
        return k0 + cp_k < K ? (is_a ? kmaj_lane_off_a : kmaj_lane_off_b) + (uint32_t)k0
                             : kOutOfRange;
    };
    auto issue_one = [&](int t, uint32_t base) {
        const int q = cw + t * NCW;
        uint32_t off;
        if constexpr (ANY_MN) {
            // base unused: each operand's own base
            const bool is_a = q < A_COPIES;
            const bool mn = is_a ? A_MN : B_MN;
            const uint32_t ld = is_a ? ROWB_A : ROWB_B;
            const uint32_t b0 = copy_base_op(mn, is_a);
            const uint32_t row = mn ? mn_row_off(t, ld)
                                    : (uint32_t)((q < A_COPIES ? q : q - A_COPIES) * RPC) * ld;
            off = b0 == kOutOfRange ? kOutOfRange : b0 + row;
            copy16_to_lds_asm(is_a ? ra : rb, lds + (fu % S) * STAGE + q * 1024, off);
            (void)base;
            return;
        }
        if constexpr (FP6)
            off = base != kOutOfRange && base + cb6[t % NOFF] < ROWB ? base + off6[t % NOFF]
                                                                    : kOutOfRange;
        else
            off = base + copy_row_off(t);
        copy16_to_lds(q < A_COPIES ? ra : rb, lds + (fu % S) * STAGE + q * 1024, off);
    };
    auto issue_finish = [&]() {
        char* st = lds + (fu % S) * STAGE;
        if constexpr (SC_LDS) {
            // wave w copies the words of A rows 64 w .. (w < 4) or of B rows
            // 64 (w - 4) ..; rows past M or N read as zero
            const uint32_t word = (uint32_t)(fc.kk * (BK / 32)) & ~3u;
            const uint32_t off = fu < T ? sc_lane_off + word : kOutOfRange;
            if constexpr (ANY_MN)
                copy4_to_lds_asm(wave < 4 ? rsa : rsb, st + DATA + wave * 256, off);
            else
                copy4_to_lds(wave < 4 ? rsa : rsb, st + DATA + wave * 256, off);
        }
        if (++fc.kk == p.ksteps) {
            fc.kk = 0;
            if (++fc.tl < my_tiles) {
                locate(fc);
                feed_resources();
            }
        }
        ++fu;
    };
    auto issue = [&]() {
        const uint32_t base = copy_base();
#pragma unroll
        for (int t = 0; t < PW; ++t) issue_one(t, base);
        issue_finish();
    };

    // ---- fragments of one unit -------------------------------------------------
    const int xr = (l32 >> SWZ) & (CPR - 1);
    // FP6: byte of chunk 0 of row R in the row-major layout; the block of
    // half-wave hi is chunk 2 hi (16 bytes) and half hi of chunk 1 (8 bytes)
    auto fp6_row = [&](int R) -> uint32_t { return (uint32_t)(R * RB); };
    const uint32_t a_frag = FP6 ? fp6_row(grp * WTM + l32) : (uint32_t)(grp * WTM + l32) * RB;
    const uint32_t b_frag = (uint32_t)A_BYTES +
                            (FP6 ? fp6_row(sub * WTN + l32) : (uint32_t)(sub * WTN + l32) * RB);
    // distance between fragment blocks of 32 rows
    constexpr uint32_t FRAG_STRIDE = 32 * RB;
    typedef typename Op::frag_t frag_t;
    frag_t fa[KSTEPS][FM], fb[KSTEPS][FN];
    auto read_frag = [&](const char* base, int s) -> frag_t {
        frag_t f;
        if constexpr (FP6) {
            // K step s holds blocks 2s and 2s + 1, chunks 3s .. 3s + 2: block
            // 2s is chunk 3s then the low half of chunk 3s + 1, block 2s + 1
            // the high half of chunk 3s + 1 then chunk 3s + 2.  The middle
            // chunk is read whole (16 bytes) and its half picked in
            // registers: 8-byte reads are served 32 lanes at a time, and rows
            // r and r + 16 of 48-byte rows share banks.
            const i32x4_t c16 = *(const i32x4_t*)(base + 16 * (3 * s + 2 * hi));
            const i32x4_t mid = *(const i32x4_t*)(base + 16 * (3 * s + 1));
            const int m0 = hi ? mid[2] : mid[0], m1 = hi ? mid[3] : mid[1];
            f = hi ? (i32x8_t){m0, m1, c16[0], c16[1], c16[2], c16[3], 0, 0}
                   : (i32x8_t){c16[0], c16[1], c16[2], c16[3], m0, m1, 0, 0};
        } else if constexpr (EBITS == 4) {
            // MXFP4: half-wave hi holds block hi of the MFMA's 64 K values,
            // the 16-byte chunk 2s + hi of the row
            f = *(const frag_t*)(base + (((2 * s + hi) ^ xr) * 16));
        } else if constexpr (CPL == 1) {
            f = *(const frag_t*)(base + (((2 * s + hi) ^ xr) * 16));
        } else {
            // scaled MFMA: block 0 of the 64 K values in bytes 0..15 of both
            // half-waves, block 1 in bytes 16..31
            i32x4_t lo = *(const i32x4_t*)(base + (((4 * s + hi) ^ xr) * 16));
            i32x4_t up = *(const i32x4_t*)(base + (((4 * s + 2 + hi) ^ xr) * 16));
            f = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        return f;
    };
    // M/N-major regions (256-byte k rows): lane 16 g + t reads k row
    // 16 (g / 2) + t / 2 (+ 0, 8, 32, 40), columns c + 16 (g % 2) + 8 (t % 2),
    // the row's swizzle 2 (k % 8) = 2 (t / 2) folded in (see the 4-wave kernel)
    const int g16 = lane >> 4, t16 = lane & 15;
    auto mn_frag = [&](int col_byte) -> uint32_t {
        return (uint32_t)((16 * (g16 >> 1) + (t16 >> 1)) * 256 + (col_byte ^ (16 * (t16 & 14))) +
                          16 * (g16 & 1) + 8 * (t16 & 1));
    };
    auto read_frag_mn = [&](const char* at) -> frag_t {
        if constexpr (ANY_MN) {
            const i32x2_t q0 = lds_read_tr8(at), q1 = lds_read_tr8(at + 8 * 256);
            const i32x2_t q2 = lds_read_tr8(at + 32 * 256), q3 = lds_read_tr8(at + 40 * 256);
            const i32x4_t lo = __builtin_shufflevector(q0, q1, 0, 1, 2, 3);
            const i32x4_t up = __builtin_shufflevector(q2, q3, 0, 1, 2, 3);
            return __builtin_bit_cast(frag_t, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            return frag_t{};
        }
    };
    // PAIR6: the operands of both K steps of a 32-row block.  Lane half hi
    // takes blocks 2 hi (step 0) and 2 hi + 1 (step 1): bytes 48 hi .. +23
    // and 48 hi + 24 .. +23 of the row, i.e. chunk 3 hi, the middle chunk
    // 3 hi + 1 (its low half ends step 0's operand, its high half starts
    // step 1's) and chunk 3 hi + 2.
    auto read_pair6 = [&](const char* base, frag_t& f0, frag_t& f1) {
        if constexpr (PAIR6) {
            const int sw = (l32 >> 3) & 1;  // the row's swizzle (blocks start at multiples of 32 rows)
            const i32x4_t x = *(const i32x4_t*)(base + 16 * ((3 * hi) ^ sw));
            const i32x4_t y = *(const i32x4_t*)(base + 16 * ((3 * hi + 1) ^ sw));
            const i32x4_t z = *(const i32x4_t*)(base + 16 * ((3 * hi + 2) ^ sw));
            f0 = (i32x8_t){x[0], x[1], x[2], x[3], y[0], y[1], 0, 0};
            f1 = (i32x8_t){y[2], y[3], z[0], z[1], z[2], z[3], 0, 0};
        }
    };
    auto read_unit = [&](int u) {
        const char* st = lds + (u % S) * STAGE;
        if constexpr (PAIR6) {
#pragma unroll
            for (int i = 0; i < FM; ++i) read_pair6(st + a_frag + i * FRAG_STRIDE, fa[0][i], fa[1][i]);
#pragma unroll
            for (int jj = 0; jj < FN; ++jj)
                read_pair6(st + b_frag + jj * FRAG_STRIDE, fb[0][jj], fb[1][jj]);
            return;
        }
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[s][i] = A_MN ? read_frag_mn(st + mn_frag(grp * WTM + 32 * i))
                                : read_frag(st + a_frag + i * FRAG_STRIDE, s);
#pragma unroll
            for (int jj = 0; jj < FN; ++jj)
                fb[s][jj] = B_MN ? read_frag_mn(st + A_BYTES + mn_frag(sub * WTN + 32 * jj))
                                 : read_frag(st + b_frag + jj * FRAG_STRIDE, s);
        }
    };

    // ---- MX scales of one unit: byte 2s of the register serves K step s ---------
    int sc_a[Op::kScaled ? FM : 1], sc_b[Op::kScaled ? FN : 1];
    // chunk mode: the 8 scale bytes a lane needs from its row's 16 (blocks
    // 2 k + hi, k = unit within the chunk), byte k of a 64-bit value
    uint64_t pk[SC_CHUNK && !PAIR6 ? FM + FN : 1];
    auto load_scales = [&](const TileCursor& c, int u) {
        if constexpr (SC_CHUNK && PAIR6) {
            // word k (unit k of the chunk: blocks 4 k .. 4 k + 3) of each
            // fragment row's 16 bytes, read afresh every unit (holding a
            // chunk's bytes in registers would not fit beside the paired
            // fragments): bytes 2 hi and 2 hi + 1 serve the two K steps
            const int k = u % UPC;
            const char* sc = lds + S * STAGE + ((u / UPC) & 1) * CHUNK_BYTES;
#pragma unroll
            for (int f = 0; f < FM + FN; ++f) {
                const bool is_a = f < FM;
                const int idx = is_a ? f : f - FM;
                const int row = (is_a ? grp * WTM : BM + sub * WTN) + idx * 32 + l32;
                const int v = (int)(*(const uint32_t*)(sc + row * 16 + 4 * k) >> (16 * hi));
                if (is_a) sc_a[idx] = v; else sc_b[idx] = v;
            }
        } else if constexpr (SC_CHUNK) {
            const int k = u % UPC;  // unit within the chunk
            if (k == 0) {
                // first unit of a chunk: one 16-byte read per fragment row
                // (16 consecutive rows per 16 lanes: no bank conflicts), bytes
                // hi, 2 + hi, 4 + hi, 6 + hi of each pair of words kept
                const char* sc = lds + S * STAGE + ((u / UPC) & 1) * CHUNK_BYTES;
                const uint32_t sel = 0x06040200u + 0x01010101u * (uint32_t)hi;
#pragma unroll
                for (int f = 0; f < FM + FN; ++f) {
                    const bool is_a = f < FM;
                    const int idx = is_a ? f : f - FM;
                    const int row = (is_a ? grp * WTM : BM + sub * WTN) + idx * 32 + l32;
                    const i32x4_t g = *(const i32x4_t*)(sc + row * 16);
                    const uint32_t lo = __builtin_amdgcn_perm((uint32_t)g[1], (uint32_t)g[0], sel);
                    const uint32_t up = __builtin_amdgcn_perm((uint32_t)g[3], (uint32_t)g[2], sel);
                    pk[f] = ((uint64_t)up << 32) | lo;
                }
            }
#pragma unroll
            for (int f = 0; f < FM + FN; ++f) {
                // byte s of v serves K step s
                const int v = (int)(uint32_t)(pk[f] >> (8 * KSTEPS * k));
                if (f < FM) sc_a[f] = v; else sc_b[f - FM] = v;
            }
        } else if constexpr (SC_LDS) {
            const char* sc = lds + (u % S) * STAGE + DATA;
            const int sh = 8 * (((c.kk * (BK / 32)) & 3) + (PAIR6 ? 2 * hi : hi));
#pragma unroll
            for (int f = 0; f < FM + FN; ++f) {
                const bool is_a = f < FM;
                const int idx = is_a ? f : f - FM;
                const int row = (is_a ? grp * WTM : BM + sub * WTN) + idx * 32 + l32;
                const int v = (int)(*(const uint32_t*)(sc + row * 4) >> sh);
                if (is_a) sc_a[idx] = v; else sc_b[idx] = v;
            }
        } else if constexpr (Op::kScaled) {
            const int kb0 = c.kk * (BK / 32);
#pragma unroll
            for (int f = 0; f < FM + FN; ++f) {
                const bool is_a = f < FM;
                const int idx = is_a ? f : f - FM;
                const int lim = is_a ? p.M : p.N;
                int row = (is_a ? c.tm * BM + grp * WTM : c.tn * BN + sub * WTN) + idx * 32 + l32;
                row = min(row, lim - 1);
                const uint8_t* src = (const uint8_t*)(is_a ? p.SA : p.SB) + (int64_t)row * kblocks;
                int v;
                if constexpr (SCALE_WORDS) {
                    // rows of K/32 bytes are whole words: the unit's bytes sit in one word
                    uint32_t w = *(const uint32_t*)(src + (kb0 & ~3));
                    v = (int)(w >> (8 * ((kb0 & 3) + (PAIR6 ? 2 * hi : hi))));
                } else {
                    int q0 = kb0 + (PAIR6 ? 2 * hi : hi);
                    v = q0 < kblocks ? src[q0] : 127;
                    if constexpr (KSTEPS > 1) {
                        int q2 = PAIR6 ? q0 + 1 : kb0 + 2 + hi;
                        v |= (q2 < kblocks ? src[q2] : 127) << (PAIR6 ? 8 : 16);
                    }
                }
                if (is_a) sc_a[idx] = v; else sc_b[idx] = v;
            }
        }
    };

    // ---- MFMAs of one unit --------------------------------------------------------
    f32x16_t acc[FM][FN];
    auto compute = [&](auto ZERO) {
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    f32x16_t c;
                    if constexpr (decltype(ZERO)::value) {
                        if (s == 0) c = (f32x16_t){};
                        else c = acc[i][j];
                    } else {
                        c = acc[i][j];
                    }
                    if constexpr (Op::kScaled) {
                        // the second K step's scale: byte 1 of a packed chunk
                        // value or of any PAIR6 form, byte 2 of the others
                        constexpr int SEL1 = (SC_CHUNK || PAIR6) ? 1 : 2;
                        if (s == 0)
                            acc[i][j] = Op::template mma<0>(fb[s][j], fa[s][i], c, sc_b[j], sc_a[i]);
                        else
                            acc[i][j] = Op::template mma<SEL1>(fb[s][j], fa[s][i], c, sc_b[j], sc_a[i]);
                    } else {
                        acc[i][j] = Op::mma(fb[s][j], fa[s][i], c);
                    }
                }
    };

    // ---- epilogue of this wave's 128 x 64 block --------------------------------
    auto epilogue = [&](const TileCursor& c) {
        char* Cb = (char*)p.C + c.batch * p.stride_c;
        const int row0 = c.tm * BM + grp * WTM;
        const int col0 = c.tn * BN + sub * WTN;
        const bool full = c.tm * BM + BM <= p.M && c.tn * BN + BN <= p.N;
        if constexpr (EPI_LDS) {
            if (full && p.N % (16 / (int)sizeof(TOut)) == 0) {
                // each block of STG_ROWS rows: MFMA layout -> staging ->
                // whole row pieces (lane l holds row l % 32 of a 32-row block)
                constexpr int CHK = STG_ROWB / 16;
                constexpr int RPI = kWaveSize * 16 / STG_ROWB;
                char* stg = lds + RING + wave * STG_BYTES;
                const int srow = l32 % STG_ROWS;
#pragma unroll
                for (int i = 0; i < FM; ++i) {
#pragma unroll
                    for (int h = 0; h < 32 / STG_ROWS; ++h) {
                        if (STG_ROWS == 32 || l32 / STG_ROWS == h) {
#pragma unroll
                            for (int j = 0; j < FN; ++j)
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const f32x16_t& a4 = acc[i][j];
                                    const int byte = (j * 32 + 8 * q + 4 * hi) * (int)sizeof(TOut);
                                    const int chunk = (byte / 16) ^ (srow & (CHK - 1));
                                    store4<TOut>(
                                        (TOut*)(stg + srow * STG_ROWB + chunk * 16 + byte % 16),
                                        a4[4 * q], a4[4 * q + 1], a4[4 * q + 2], a4[4 * q + 3]);
                                }
                        }
                        wave_lds_exchange();
#pragma unroll
                        for (int t = 0; t < STG_ROWS / RPI; ++t) {
                            const int r = t * RPI + lane / CHK;
                            const int ck = lane % CHK;
                            const i32x4_t d = *(const i32x4_t*)(stg + r * STG_ROWB +
                                                                ((ck ^ (r & (CHK - 1))) * 16));
                            char* g = Cb +
                                      ((int64_t)(row0 + i * 32 + h * STG_ROWS + r) * p.N + col0) *
                                          (int64_t)sizeof(TOut) +
                                      ck * 16;
                            *(i32x4_t*)g = d;
                        }
                        wave_lds_exchange();
                    }
                }
                return;
            }
        }
        const bool vec = (p.N & 3) == 0;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = row0 + i * 32 + l32;
            if (m >= p.M) continue;
            TOut* row = (TOut*)Cb + (int64_t)m * p.N;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = col0 + j * 32 + 8 * q + 4 * hi;
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
    };

    // ---- prologue: units 0 .. S-2 resident -------------------------------------------
    locate(fc);
    feed_resources();
    if constexpr (SC_CHUNK) {
        locate(scc);
        chunk_resources();
        issue_chunk();  // chunk 0; chunk c + 1 follows in the memory halves of unit UPC c
    }
#pragma unroll
    for (int u = 0; u < S - 1; ++u) issue();
    wait_vmcnt<0>();
    barrier_lds();

    // ---- half-periods -------------------------------------------------------------
    // Group 0 reads unit u in half 2u-1 and computes it in half 2u; group 1
    // reads it in half 2u and computes it in half 2u+1.  Each group runs one
    // plain loop -- memory half, barrier, MFMA half, barrier -- group 1 one
    // half behind, so both execute 2T + 2 barriers.  The memory half of unit
    // u also issues this wave's copies of unit u + S - 1.
    auto run = [&](auto GROUP0) {
        constexpr bool G0 = decltype(GROUP0)::value;
        TileCursor cc = {0, 0, 0, 0, 0};
        locate(cc);
        if constexpr (!G0) __builtin_amdgcn_s_barrier();  // half -1: group 0 reads unit 0
        for (int u = 0; u < T; ++u) {
            // ---- memory half
            if (u > 0 && cc.kk == 0) {
                // the previous unit finished a tile: convert and store it
                // while the other group computes
                TileCursor ec = {cc.tl - 1, 0, 0, 0, 0};
                locate(ec);
                epilogue(ec);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (Op::kScaled) load_scales(cc, u);
            read_unit(u);
            if constexpr (SC_CHUNK) {
                // the other buffer held the chunk before this one, which both
                // groups finished reading in earlier halves
                if (u == cu - UPC) issue_chunk();
            }
            issue();
            // Waits before the barrier.  Scales loaded to registers precede
            // this half's copies, and loads return in order, so vmcnt(OPS)
            // covers them.  Group 1's copies of unit u + 1, which group 0 reads
            // in the next half, have (S - 2) * OPS operations issued after
            // them.
            constexpr bool REG_SCALES = Op::kScaled && !SC_LDS && !SC_CHUNK;
            if constexpr (G0) {
                if constexpr (REG_SCALES) wait_vmcnt<OPS>();
            } else if constexpr (REG_SCALES) {
                wait_vmcnt<OPS>();
            } else {
                wait_vmcnt<(S - 2) * OPS>();
            }
            barrier_lds();
            // ---- MFMA half
            if (cc.kk == 0)
                compute(std::true_type{});
            else
                compute(std::false_type{});
            advance(cc);
            // group 0's share of unit u + 1 lands before its next memory half
            if constexpr (G0) wait_vmcnt<(S - 2) * OPS>();
            __builtin_amdgcn_s_barrier();
        }
        // epilogue of the last tile, then the halves that keep barrier counts equal
        TileCursor ec = {my_tiles - 1, 0, 0, 0, 0};
        locate(ec);
        epilogue(ec);
        barrier_lds();
        if constexpr (G0) __builtin_amdgcn_s_barrier();
    };
    if (grp == 0)
        run(std::true_type{});
    else
        run(std::false_type{});
}

}  // namespace tcm
