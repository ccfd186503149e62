// C ABI of libtcm: argument validation, planning and dispatch.  Every
// argument is checked on the host before any HIP call, in this order: dtype
// pair, sizes, pointers, supported range, alignment.
#include <limits.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/tcm.h"
#include "tcm_internal.h"

namespace tcm {

VariantInfo variant_info(int32_t v) {
    switch (v) {
    case V_T128x256: return {128, 256, 64, 2, 1, 16, kThreads};
    case V_T128x128: return {128, 128, 64, 2, 2, 16, kThreads};
    case V_T128x64: return {128, 64, 64, 2, 3, 16, kThreads};
    case V_MX128x128: return {128, 128, 128, 2, 1, 8, kThreads};
    case V_T256x256_SPLIT3: return {256, 256, 64, 2, 1, 16, kThreads};
    case V_T256x256_M16: return {256, 256, 64, 2, 1, 16, kThreads};
    case V_MX16_256: return {256, 256, 128, 2, 1, 8, kThreads};
    case V_MX4_16_256: return {256, 256, 256, 2, 1, 4, kThreads};
    // MXFP6 on the 16x16 kernel: 96-byte rows in 128-byte LDS rows
    case V_MX6_16_256: return {256, 256, 128, 2, 1, 6, kThreads};
    case V_MXPP256_K64S4: return {256, 256, 64, 4, 1, 8, 512};
    case V_MX4PP256: return {256, 256, 128, 4, 1, 4, 512};
    case V_MX6PP256: return {256, 256, 64, 4, 1, 6, 512};
    case V_MX6PP256_K128: return {256, 256, 128, 3, 1, 6, 512};
    // NVFP4: the LDS tiles hold fp16
    case V_NV4_256: return {256, 256, 64, 2, 1, 16, kThreads};
    case V_NV4_128: return {128, 128, 64, 2, 2, 16, kThreads};
    case V_NV4W_256: return {256, 256, 64, 2, 1, 16, kThreads};
    case V_NV4W_128: return {128, 128, 64, 2, 2, 16, kThreads};
    // NVFP4 on the 16x16 kernel: E2M1 rows in LDS
    case V_NV4_16_256: return {256, 256, 256, 2, 1, 4, kThreads};
    case V_MX256x128: return {256, 128, 128, 2, 1, 8, kThreads};
    }
    return {0, 0, 0, 0, 0, 0, kThreads};
}

}  // namespace tcm

namespace {

using namespace tcm;

constexpr int64_t kMaxK = int64_t(1) << 20;     // keeps buffer offsets within 32 bits
constexpr int64_t kMaxMN = int64_t(1) << 30;    // row indices stay in int32
constexpr int64_t kMaxLd = int64_t(1) << 21;    // operand leading dimensions (32-bit offsets)
constexpr int kMaxDevices = 64;

struct DeviceInfo {
    int cus = 0;
    bool gfx950 = false;
    hipError_t err = hipSuccess;
};

DeviceInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

tcm_status device_info(DeviceInfo* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TCM_ERR_NO_DEVICE;
    std::call_once(g_dev_once[dev], [dev] {
        hipDeviceProp_t prop;
        DeviceInfo& d = g_dev[dev];
        d.err = hipGetDeviceProperties(&prop, dev);
        if (d.err == hipSuccess) {
            d.cus = prop.multiProcessorCount;
            d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        }
    });
    *out = g_dev[dev];
    if (out->err != hipSuccess || !out->gfx950 || out->cus <= 0) return TCM_ERR_NO_DEVICE;
    return TCM_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool mul_ok(int64_t a, int64_t b, int64_t c) {
    int64_t t;
    return !__builtin_mul_overflow(a, b, &t) && !__builtin_mul_overflow(t, c, &t) &&
           t < (int64_t(1) << 62);
}

int elem_bytes(tcm_dtype d) {
    switch (d) {
    case TCM_F16:
    case TCM_BF16: return 2;
    case TCM_F32: return 4;
    case TCM_E4M3:
    case TCM_E8M0: return 1;
    case TCM_E2M1:
    case TCM_E2M3:
    case TCM_E3M2: return 0;  // packed below a byte
    }
    return 0;
}

// Sizes shared by every entry point.  *empty is set when there is nothing to
// write (batch, M or N is zero).
tcm_status check_sizes(int64_t batch, int64_t M, int64_t N, int64_t K, bool* empty) {
    if (batch < 0 || M < 0 || N < 0 || K < 0) return TCM_ERR_INVALID_SHAPE;
    if (!mul_ok(batch, M, K) || !mul_ok(batch, N, K) || !mul_ok(batch, M, N))
        return TCM_ERR_INVALID_SHAPE;
    *empty = batch == 0 || M == 0 || N == 0;
    return TCM_OK;
}

tcm_status check_range(int64_t batch, int64_t M, int64_t N, int64_t K) {
    if (K > kMaxK || M > kMaxMN || N > kMaxMN) return TCM_ERR_UNSUPPORTED_SHAPE;
    // tile counts with the smallest tile must fit in int32
    if (batch * cdiv(M, 128) * cdiv(N, 64) > INT32_MAX) return TCM_ERR_UNSUPPORTED_SHAPE;
    return TCM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_nv4_variant(int32_t v) {
    return v == V_NV4_256 || v == V_NV4_128 || v == V_NV4W_256 || v == V_NV4W_128 ||
           v == V_NV4_16_256;
}

// variants launched only by their own entry point (not forceable elsewhere)
bool own_entry_variant(int32_t v) { return is_nv4_variant(v) || v == V_MX256x128; }

// TCM_FORCE_VARIANT=<id> (read at every call) forces a kernel variant of the
// matching family, for tuning sweeps and per-variant tests; unset or invalid,
// the heuristic below chooses.
int32_t forced_variant() {
    const char* e = getenv("TCM_FORCE_VARIANT");
    return e && *e ? (int32_t)atoi(e) : (int32_t)-1;
}

// TCM_MAX_GRID=<n> (read at every call) caps the number of persistent
// workgroups, so that small problems also run several tiles per workgroup
// (tests of the tile hand-over); unset or not positive, the grid is
// min(tiles, CUs x occupancy).
int64_t max_grid() {
    const char* e = getenv("TCM_MAX_GRID");
    const long long g = e && *e ? atoll(e) : 0;
    return g > 0 ? (int64_t)g : INT64_MAX;
}

// TCM_GROUP_M=<n> (read at every call) sets the tile rows per group of the
// grouped tile order (tuning sweeps); unset or not positive, 4.
int32_t group_m() {
    const char* e = getenv("TCM_GROUP_M");
    const long g = e && *e ? atol(e) : 0;
    return g > 0 && g <= 1024 ? (int32_t)g : 4;
}

// Tile choice: the largest tile whose tile count still gives every CU at
// least one tile with little padding; small problems take the smallest tile.
// Families by element bits: 16 (f16/bf16), 8 (MXFP8), 6 (MXFP6), 4 (MXFP4).
int32_t choose_variant(int64_t batch, int64_t M, int64_t N, int32_t bits, int cus) {
    const int32_t f = forced_variant();
    if (f >= 0 && variant_info(f).tile_m > 0 && variant_info(f).elem_bits == bits &&
        !own_entry_variant(f))
        return f;
    static const int32_t plain[] = {V_T256x256_M16, V_T128x256, V_T128x128, V_T128x64};
    static const int32_t mxv[] = {V_MXPP256_K64S4, V_MX128x128};
    static const int32_t mx4[] = {V_MX4PP256};
    static const int32_t mx6[] = {V_MX6PP256_K128};
    const int32_t* cand = bits == 8 ? mxv : bits == 4 ? mx4 : bits == 6 ? mx6 : plain;
    const int n = bits == 8 ? 2 : bits == 4 ? 1 : bits == 6 ? 1 : 4;
    for (int i = 0; i < n; ++i) {
        VariantInfo vi = variant_info(cand[i]);
        int64_t tiles = batch * cdiv(M, vi.tile_m) * cdiv(N, vi.tile_n);
        double fill = double(batch) * M * N / (double(tiles) * vi.tile_m * vi.tile_n);
        if (tiles >= cus && fill >= 0.9) return cand[i];
    }
    return cand[n - 1];
}

// Variants the C-input epilogue kernels run (gemm_epi.hip): the 128-row
// tiles as chosen, every other 16-bit choice as the 256 x 256 split-3 form.
int32_t epi_variant(int32_t v) {
    return (v == V_T128x256 || v == V_T128x128 || v == V_T128x64) ? v : V_T256x256_SPLIT3;
}

// Variants with an M-major A or N-major B (gemm_mn.h): 256 x 256 split-3 for
// 256-row choices, 128 x 128 otherwise (its 256-byte M/N rows are the
// narrowest the transposing reads' bank spread allows).
int32_t mn_variant(int32_t v) {
    return variant_info(v).tile_m == 256 ? V_T256x256_SPLIT3 : V_T128x128;
}

tcm_status plan_variant(int32_t v, int64_t batch, int64_t M, int64_t N, int64_t K, int cus,
                        tcm_plan* plan, GemmArgs* args) {
    VariantInfo vi = variant_info(v);
    int64_t tm = cdiv(M, vi.tile_m), tn = cdiv(N, vi.tile_n);
    int64_t tiles = batch * tm * tn;
    int64_t slots = int64_t(cus) * vi.occupancy;
    int64_t grid = tiles < slots ? tiles : slots;
    const int64_t cap = max_grid();
    if (grid > cap) grid = cap;
    // (the 16x16 MXFP6 kernel keeps each 96-byte row slice in 128 LDS bytes)
    const int32_t lds_bits = v == V_MX6_16_256 ? 8 : vi.elem_bits;
    int32_t stage = (vi.tile_m + vi.tile_n) * vi.tile_k * lds_bits / 8;
    if (plan) {
        plan->tile_m = vi.tile_m;
        plan->tile_n = vi.tile_n;
        plan->tile_k = vi.tile_k;
        plan->stages = vi.stages;
        plan->threads = vi.threads;
        plan->stage_bytes = stage;
        plan->lds_bytes = stage * vi.stages;
        plan->grid = (int32_t)grid;
        plan->tiles = tiles;
        plan->kernel = v;
    }
    if (args) {
        memset(args, 0, sizeof(*args));
        args->M = (int32_t)M;
        args->N = (int32_t)N;
        args->K = (int32_t)K;
        args->batch = (int32_t)batch;
        args->tiles_m = (int32_t)tm;
        args->tiles_n = (int32_t)tn;
        args->tiles_per_batch = (int32_t)(tm * tn);
        args->total_tiles = (int32_t)tiles;
        args->ksteps = K > 0 ? (int32_t)cdiv(K, vi.tile_k) : 1;
        args->group_m = group_m();
        // dense storage unless the caller says otherwise
        args->lda = args->ldb = (int32_t)K;
        args->ldc = args->ldcin = (int32_t)N;
    }
    return TCM_OK;
}

tcm_status make_plan(int64_t batch, int64_t M, int64_t N, int64_t K, int32_t bits, int cus,
                     tcm_plan* plan, GemmArgs* args) {
    return plan_variant(choose_variant(batch, M, N, bits, cus), batch, M, N, K, cus, plan, args);
}

// NVFP4: the 256 x 256 tile where it fills the CUs with little padding; a
// row's scales of four slices in one 16-byte load where K and the scale
// tensors allow it (wide).
// MXFP6: the 128-deep kernel reads its scales as 32-bit words or 16-byte
// pieces (K a multiple of 128, word-aligned scale tensors); with scales read
// byte by byte it would spill registers, so such calls take the 64-deep
// kernel unless a variant is forced.  Where scales come as 16-byte pieces
// (K % 512 == 0, 16-byte aligned scale tensors) the 16 x 16 x 128 kernel
// (variant 36) takes the 128-deep kernel's place unless that one is forced.
int32_t mx6_variant(int32_t v, bool scale_words, bool scale_chunks) {
    if (v == V_MX6_16_256 && !scale_chunks) v = V_MX6PP256_K128;
    if (v == V_MX6PP256_K128 && scale_chunks && forced_variant() != V_MX6PP256_K128) return V_MX6_16_256;
    return v == V_MX6PP256_K128 && !scale_words && forced_variant() != V_MX6PP256_K128 ? V_MX6PP256 : v;
}

// MXFP8 256 x 256 tiles: the 16 x 16 x 128 kernel (variant 31) where scales
// can be read as 16-byte pieces (K % 512 == 0, 16-byte aligned scale
// tensors), the ping-pong kernel (variant 14) elsewhere or when forced.
int32_t mx8_variant(int32_t v, bool scale_chunks) {
    if (v == V_MX16_256 && !scale_chunks) return V_MXPP256_K64S4;
    if (v == V_MXPP256_K64S4 && scale_chunks && forced_variant() != V_MXPP256_K64S4) return V_MX16_256;
    return v;
}

// MXFP4 256 x 256 tiles, the same way: the 16 x 16 x 128 kernel (variant 32)
// with 16-byte scale pieces, the ping-pong kernel (variant 20) elsewhere or
// when forced.
int32_t mx4_variant(int32_t v, bool scale_chunks) {
    if (v == V_MX4_16_256 && !scale_chunks) return V_MX4PP256;
    if (v == V_MX4PP256 && scale_chunks && forced_variant() != V_MX4PP256) return V_MX4_16_256;
    return v;
}

int32_t nv4_variant(int64_t M, int64_t N, bool wide, int cus) {
    const int64_t tiles = cdiv(M, 256) * cdiv(N, 256);
    const double fill = double(M) * N / (double(tiles) * 256 * 256);
    const bool big = tiles >= cus && fill >= 0.9;
    int32_t v = wide ? (big ? V_NV4_16_256 : V_NV4W_128) : (big ? V_NV4_256 : V_NV4_128);
    const int32_t f = forced_variant();
    if (f == V_NV4_256 || f == V_NV4_128 ||
        (wide && (f == V_NV4W_256 || f == V_NV4W_128 || f == V_NV4_16_256)))
        v = f;
    return v;
}

// MXFP8 in other arrangements.  With an M/N-major operand, dense output
// rows and every k row's offset within 32 bits (K * ld), the ping-pong
// kernel's 256 x 256 tiles where they fill the CUs; otherwise the 4-wave
// kernel's 256 x 128 tiles where they do, else 128 x 128.
int32_t mx_mn_variant(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldo,
                      bool any_mn, int cus) {
    auto fills = [&](int64_t tm, int64_t tn) {
        const int64_t tiles = cdiv(M, tm) * cdiv(N, tn);
        return tiles >= cus && double(M) * N / (double(tiles) * tm * tn) >= 0.9;
    };
    const int64_t lim = (int64_t(1) << 31) - 256;
    const bool pp = any_mn && ldo == N && K * lda < lim && K * ldb < lim;
    int32_t v = pp && fills(256, 256) ? V_MXPP256_K64S4
                : fills(256, 128)     ? V_MX256x128
                                      : V_MX128x128;
    const int32_t f = forced_variant();
    if (f == V_MX256x128 || f == V_MX128x128 || (pp && f == V_MXPP256_K64S4)) v = f;
    return v;
}

bool plain_pair(tcm_dtype in, tcm_dtype out) {
    return (in == TCM_F16 || in == TCM_BF16) && (out == TCM_F32 || out == TCM_BF16);
}

tcm_status run_plain(const void* A, const void* B, void* Out, int64_t batch, int64_t M, int64_t N,
                     int64_t K, tcm_dtype dtype, tcm_dtype out_dtype, void* stream) {
    if (!plain_pair(dtype, out_dtype)) return TCM_ERR_UNSUPPORTED_DTYPE;
    bool empty = false;
    tcm_status s = check_sizes(batch, M, N, K, &empty);
    if (s != TCM_OK || empty) return s;
    if (!Out || (K > 0 && (!A || !B))) return TCM_ERR_NULL_POINTER;
    if ((s = check_range(batch, M, N, K)) != TCM_OK) return s;
    const int es = elem_bytes(dtype);
    if ((A && !aligned16(A)) || (B && !aligned16(B)) || !aligned16(Out) || (K * es) % 16 != 0)
        return TCM_ERR_MISALIGNED;
    DeviceInfo dev;
    if ((s = device_info(&dev)) != TCM_OK) return s;
    tcm_plan plan;
    GemmArgs a;
    make_plan(batch, M, N, K, 16, dev.cus, &plan, &a);
    a.A = A;
    a.B = B;
    a.C = Out;
    a.stride_a = M * K * es;
    a.stride_b = N * K * es;
    a.stride_c = M * N * elem_bytes(out_dtype);
    hipError_t e = launch_gemm_tn(plan.kernel, (int32_t)dtype, (int32_t)out_dtype, a, plan.grid,
                                  (hipStream_t)stream);
    return e == hipSuccess ? TCM_OK : TCM_ERR_HIP;
}

}  // namespace

extern "C" {

tcm_status tcm_gemm_tn(const void* A, const void* B, void* Out, int64_t M, int64_t N, int64_t K,
                       tcm_dtype dtype, tcm_dtype out_dtype, void* stream) {
    return run_plain(A, B, Out, 1, M, N, K, dtype, out_dtype, stream);
}

tcm_status tcm_batched_gemm_tn(const void* A, const void* B, void* Out, int64_t batch, int64_t M,
                               int64_t N, int64_t K, tcm_dtype dtype, tcm_dtype out_dtype,
                               void* stream) {
    return run_plain(A, B, Out, batch, M, N, K, dtype, out_dtype, stream);
}

}  // extern "C"

namespace {

// The MX entry points: elements of `bits` bits (8 = E4M3, 6 = E2M3 or E3M2 as
// elem_dtype says, 4 = E2M1 pairs).
tcm_status run_mx(int32_t bits, const void* A, const void* B, const void* scale_A,
                  const void* scale_B, void* Out, int64_t M, int64_t N, int64_t K,
                  tcm_dtype out_dtype, void* stream, tcm_dtype elem_dtype = TCM_E4M3) {
    if (!(out_dtype == TCM_F32 || out_dtype == TCM_BF16)) return TCM_ERR_UNSUPPORTED_DTYPE;
    if (bits == 6 && !(elem_dtype == TCM_E2M3 || elem_dtype == TCM_E3M2))
        return TCM_ERR_UNSUPPORTED_DTYPE;
    bool empty = false;
    tcm_status s = check_sizes(1, M, N, K, &empty);
    if (s != TCM_OK || empty) return s;
    if (!Out || (K > 0 && (!A || !B || !scale_A || !scale_B))) return TCM_ERR_NULL_POINTER;
    if ((s = check_range(1, M, N, K)) != TCM_OK) return s;
    if (K % 32 != 0) return TCM_ERR_UNSUPPORTED_SHAPE;
    // rows of K * bits / 8 bytes, whole 16-byte pieces (K % 32 == 0 suffices
    // for 8 and 4 bits; 6 bits need K % 64 == 0)
    if ((A && !aligned16(A)) || (B && !aligned16(B)) || !aligned16(Out) || (K * bits / 8) % 16 != 0)
        return TCM_ERR_MISALIGNED;
    DeviceInfo dev;
    if ((s = device_info(&dev)) != TCM_OK) return s;
    // Wide scale reads need every row's K/32 bytes to be whole words (16-byte
    // pieces) and the arrays aligned to match.
    const uintptr_t sa = reinterpret_cast<uintptr_t>(scale_A), sb = reinterpret_cast<uintptr_t>(scale_B);
    int32_t scale_mode = 0;
    if (K > 0 && K % 512 == 0 && ((sa | sb) & 15u) == 0)
        scale_mode = 2;
    else if (K > 0 && K % 128 == 0 && ((sa | sb) & 3u) == 0)
        scale_mode = 1;
    tcm_plan plan;
    GemmArgs a;
    if (bits == 6)
        plan_variant(mx6_variant(choose_variant(1, M, N, bits, dev.cus), scale_mode >= 1, scale_mode == 2),
                     1, M, N, K, dev.cus, &plan, &a);
    else if (bits == 8)
        plan_variant(mx8_variant(choose_variant(1, M, N, bits, dev.cus), scale_mode == 2), 1, M, N,
                     K, dev.cus, &plan, &a);
    else if (bits == 4)
        plan_variant(mx4_variant(choose_variant(1, M, N, bits, dev.cus), scale_mode == 2), 1, M, N,
                     K, dev.cus, &plan, &a);
    else
        make_plan(1, M, N, K, bits, dev.cus, &plan, &a);
    a.A = A;
    a.B = B;
    a.SA = scale_A;
    a.SB = scale_B;
    a.C = Out;
    a.stride_a = M * K * bits / 8;
    a.stride_b = N * K * bits / 8;
    a.stride_c = M * N * elem_bytes(out_dtype);
    hipError_t e = bits == 6 ? launch_gemm_mx6(plan.kernel, (int32_t)out_dtype, scale_mode,
                                               (int32_t)elem_dtype, a, plan.grid,
                                               (hipStream_t)stream)
                             : launch_gemm_mx(plan.kernel, (int32_t)out_dtype, scale_mode, a,
                                              plan.grid, (hipStream_t)stream);
    return e == hipSuccess ? TCM_OK : TCM_ERR_HIP;
}

}  // namespace

extern "C" {

tcm_status tcm_gemm_mx_fp8(const void* A, const void* B, const void* scale_A, const void* scale_B,
                           void* Out, int64_t M, int64_t N, int64_t K, tcm_dtype out_dtype,
                           void* stream) {
    return run_mx(8, A, B, scale_A, scale_B, Out, M, N, K, out_dtype, stream);
}

tcm_status tcm_gemm_mx_fp4(const void* A, const void* B, const void* scale_A, const void* scale_B,
                           void* Out, int64_t M, int64_t N, int64_t K, tcm_dtype out_dtype,
                           void* stream) {
    return run_mx(4, A, B, scale_A, scale_B, Out, M, N, K, out_dtype, stream);
}

tcm_status tcm_gemm_nvfp4(const void* A, const void* B, const void* scale_A, const void* scale_B,
                          float global_scale_A, float global_scale_B, void* Out, int64_t M,
                          int64_t N, int64_t K, tcm_dtype out_dtype, void* stream) {
    if (!(out_dtype == TCM_F16 || out_dtype == TCM_BF16 || out_dtype == TCM_F32))
        return TCM_ERR_UNSUPPORTED_DTYPE;
    bool empty = false;
    tcm_status s = check_sizes(1, M, N, K, &empty);
    if (s != TCM_OK || empty) return s;
    if (!Out || (K > 0 && (!A || !B || !scale_A || !scale_B))) return TCM_ERR_NULL_POINTER;
    if ((s = check_range(1, M, N, K)) != TCM_OK) return s;
    if (K % 32 != 0) return TCM_ERR_UNSUPPORTED_SHAPE;
    // rows of K/2 bytes (whole 16-byte pieces); scales read two at a time
    auto aligned2 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; };
    if ((A && !aligned16(A)) || (B && !aligned16(B)) || !aligned16(Out) ||
        (scale_A && !aligned2(scale_A)) || (scale_B && !aligned2(scale_B)))
        return TCM_ERR_MISALIGNED;
    DeviceInfo dev;
    if ((s = device_info(&dev)) != TCM_OK) return s;
    // (the wide form walks a tile's slices in pairs: K > 0)
    const bool wide = K > 0 && K % 256 == 0 && (!scale_A || aligned16(scale_A)) &&
                      (!scale_B || aligned16(scale_B));
    const int32_t v = nv4_variant(M, N, wide, dev.cus);
    tcm_plan plan;
    GemmArgs a;
    plan_variant(v, 1, M, N, K, dev.cus, &plan, &a);
    a.A = A;
    a.B = B;
    a.SA = scale_A;
    a.SB = scale_B;
    a.C = Out;
    a.stride_a = M * K / 2;
    a.stride_b = N * K / 2;
    a.stride_c = M * N * elem_bytes(out_dtype);
    a.alpha = global_scale_A * global_scale_B;
    a.beta = 0.0f;
    a.c_dtype = (int32_t)TCM_F32;
    a.op = TCM_OP_IDENTITY;
    hipError_t e = launch_gemm_nv4(v, (int32_t)out_dtype, a, plan.grid, (hipStream_t)stream);
    return e == hipSuccess ? TCM_OK : TCM_ERR_HIP;
}

tcm_status tcm_gemm_mx(const void* A, tcm_order a_order, int64_t lda, const void* B,
                       tcm_order b_order, int64_t ldb, const void* scale_A, const void* scale_B,
                       void* Out, int64_t ldo, int64_t M, int64_t N, int64_t K,
                       tcm_dtype elem_dtype, tcm_dtype out_dtype, void* stream) {
    if (elem_dtype != TCM_E4M3 || !(out_dtype == TCM_F32 || out_dtype == TCM_BF16))
        return TCM_ERR_UNSUPPORTED_DTYPE;
    bool empty = false;
    tcm_status s = check_sizes(1, M, N, K, &empty);
    if (s != TCM_OK) return s;
    auto order_ok = [](tcm_order o) { return o == TCM_ROW_MAJOR || o == TCM_COL_MAJOR; };
    if (!order_ok(a_order) || !order_ok(b_order)) return TCM_ERR_INVALID_ARGUMENT;
    const bool a_mn = a_order == TCM_COL_MAJOR;  // A's M index contiguous
    const bool b_mn = b_order == TCM_ROW_MAJOR;  // B's N index contiguous
    auto at_least = [](int64_t ld, int64_t n) { return ld >= (n > 1 ? n : 1); };
    if (!at_least(lda, a_mn ? M : K) || !at_least(ldb, b_mn ? N : K) || !at_least(ldo, N))
        return TCM_ERR_INVALID_SHAPE;
    if (!mul_ok(M, ldo, 1)) return TCM_ERR_INVALID_SHAPE;
    if (empty) return TCM_OK;
    if (!Out || (K > 0 && (!A || !B || !scale_A || !scale_B))) return TCM_ERR_NULL_POINTER;
    if ((s = check_range(1, M, N, K)) != TCM_OK) return s;
    if (lda > kMaxLd || ldb > kMaxLd || ldo > INT32_MAX || K % 32 != 0)
        return TCM_ERR_UNSUPPORTED_SHAPE;
    // stored rows of whole 16-byte pieces (16 E4M3 elements)
    if ((A && !aligned16(A)) || (B && !aligned16(B)) || !aligned16(Out) || lda % 16 != 0 ||
        ldb % 16 != 0)
        return TCM_ERR_MISALIGNED;
    // dense TN storage: the same kernels as tcm_gemm_mx_fp8
    if (!a_mn && !b_mn && lda == K && ldb == K && ldo == N)
        return run_mx(8, A, B, scale_A, scale_B, Out, M, N, K, out_dtype, stream);
    DeviceInfo dev;
    if ((s = device_info(&dev)) != TCM_OK) return s;
    const int32_t v = mx_mn_variant(M, N, K, lda, ldb, ldo, a_mn || b_mn, dev.cus);
    tcm_plan plan;
    GemmArgs a;
    plan_variant(v, 1, M, N, K, dev.cus, &plan, &a);
    a.A = A;
    a.B = B;
    a.SA = scale_A;
    a.SB = scale_B;
    a.C = Out;
    a.lda = (int32_t)lda;
    a.ldb = (int32_t)ldb;
    a.ldc = (int32_t)ldo;
    // scale rows read as 16-byte pieces (ping-pong kernel, K % 512 == 0,
    // 16-byte aligned arrays) or as words (K % 128 == 0, word-aligned), else
    // byte by byte; the 4-wave kernels read words in modes 1 and 2
    const uintptr_t sa = reinterpret_cast<uintptr_t>(scale_A), sb = reinterpret_cast<uintptr_t>(scale_B);
    const int32_t scale_mode = K > 0 && K % 512 == 0 && ((sa | sb) & 15u) == 0 ? 2
                               : K > 0 && K % 128 == 0 && ((sa | sb) & 3u) == 0 ? 1
                                                                                : 0;
    const int32_t od = (int32_t)out_dtype;
    const hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (a_mn && b_mn)
        e = launch_gemm_mx_mn<true, true>(v, od, scale_mode, a, plan.grid, st);
    else if (a_mn)
        e = launch_gemm_mx_mn<true, false>(v, od, scale_mode, a, plan.grid, st);
    else if (b_mn)
        e = launch_gemm_mx_mn<false, true>(v, od, scale_mode, a, plan.grid, st);
    else
        e = launch_gemm_mx_mn<false, false>(v, od, scale_mode, a, plan.grid, st);
    return e == hipSuccess ? TCM_OK : TCM_ERR_HIP;
}

tcm_status tcm_gemm_mx_fp6(const void* A, const void* B, const void* scale_A, const void* scale_B,
                           void* Out, int64_t M, int64_t N, int64_t K, tcm_dtype elem_dtype,
                           tcm_dtype out_dtype, void* stream) {
    return run_mx(6, A, B, scale_A, scale_B, Out, M, N, K, out_dtype, stream, elem_dtype);
}

tcm_status tcm_gemm_tn_ex(const void* A, const void* B, const void* C, void* Out, int64_t M,
                          int64_t N, int64_t K, tcm_dtype dtype, tcm_dtype c_dtype,
                          tcm_dtype out_dtype, float alpha, float beta, void* stream) {
    auto out_ok = [](tcm_dtype d) { return d == TCM_F16 || d == TCM_BF16 || d == TCM_F32; };
    if (!(dtype == TCM_F16 || dtype == TCM_BF16) || !out_ok(out_dtype) ||
        (beta != 0.0f && !out_ok(c_dtype)))
        return TCM_ERR_UNSUPPORTED_DTYPE;
    bool empty = false;
    tcm_status s = check_sizes(1, M, N, K, &empty);
    if (s != TCM_OK || empty) return s;
    if (!Out || (K > 0 && (!A || !B)) || (beta != 0.0f && !C)) return TCM_ERR_NULL_POINTER;
    if ((s = check_range(1, M, N, K)) != TCM_OK) return s;
    if ((A && !aligned16(A)) || (B && !aligned16(B)) || !aligned16(Out) ||
        (beta != 0.0f && !aligned16(C)) || (K * 2) % 16 != 0)
        return TCM_ERR_MISALIGNED;
    DeviceInfo dev;
    if ((s = device_info(&dev)) != TCM_OK) return s;
    tcm_plan plan;
    GemmArgs a;
    plan_variant(epi_variant(choose_variant(1, M, N, 16, dev.cus)), 1, M, N, K, dev.cus, &plan,
                 &a);
    a.A = A;
    a.B = B;
    a.C = Out;
    a.stride_a = M * K * 2;
    a.stride_b = N * K * 2;
    a.stride_c = M * N * elem_bytes(out_dtype);
    a.Cin = beta != 0.0f ? C : nullptr;
    a.stride_cin = beta != 0.0f ? M * N * elem_bytes(c_dtype) : 0;
    a.alpha = alpha;
    a.beta = beta;
    a.c_dtype = (int32_t)c_dtype;
    hipError_t e = launch_gemm_epi(plan.kernel, (int32_t)dtype, (int32_t)out_dtype, a, plan.grid,
                                   (hipStream_t)stream);
    return e == hipSuccess ? TCM_OK : TCM_ERR_HIP;
}

tcm_status tcm_gemm(const void* A, tcm_order a_order, int64_t lda, const void* B,
                    tcm_order b_order, int64_t ldb, const void* C, int64_t ldc, void* Out,
                    int64_t ldo, int64_t M, int64_t N, int64_t K, tcm_dtype dtype,
                    tcm_dtype c_dtype, tcm_dtype out_dtype, float alpha, float beta, tcm_op op,
                    void* stream) {
    auto out_ok = [](tcm_dtype d) { return d == TCM_F16 || d == TCM_BF16 || d == TCM_F32; };
    if (!(dtype == TCM_F16 || dtype == TCM_BF16) || !out_ok(out_dtype) ||
        (beta != 0.0f && !out_ok(c_dtype)))
        return TCM_ERR_UNSUPPORTED_DTYPE;
    bool empty = false;
    tcm_status s = check_sizes(1, M, N, K, &empty);
    if (s != TCM_OK) return s;
    auto order_ok = [](tcm_order o) { return o == TCM_ROW_MAJOR || o == TCM_COL_MAJOR; };
    if (!order_ok(a_order) || !order_ok(b_order) || (int)op < TCM_OP_IDENTITY ||
        (int)op > TCM_OP_SILU)
        return TCM_ERR_INVALID_ARGUMENT;
    // a stored row holds the matrix's columns (row-major) or its rows
    // (column-major); every leading dimension covers at least that, and 1
    const bool a_mn = a_order == TCM_COL_MAJOR;  // A's M index contiguous
    const bool b_mn = b_order == TCM_ROW_MAJOR;  // B's N index contiguous
    auto at_least = [](int64_t ld, int64_t n) { return ld >= (n > 1 ? n : 1); };
    if (!at_least(lda, a_mn ? M : K) || !at_least(ldb, b_mn ? N : K) || !at_least(ldo, N) ||
        (beta != 0.0f && !at_least(ldc, N)))
        return TCM_ERR_INVALID_SHAPE;
    if (!mul_ok(M, ldo, 1) || (beta != 0.0f && !mul_ok(M, ldc, 1))) return TCM_ERR_INVALID_SHAPE;
    if (empty) return TCM_OK;
    if (!Out || (K > 0 && (!A || !B)) || (beta != 0.0f && !C)) return TCM_ERR_NULL_POINTER;
    if ((s = check_range(1, M, N, K)) != TCM_OK) return s;
    if (lda > kMaxLd || ldb > kMaxLd || ldo > INT32_MAX || (beta != 0.0f && ldc > INT32_MAX))
        return TCM_ERR_UNSUPPORTED_SHAPE;
    // 16-byte operand rows; a K-major operand's rows end on a whole 16-byte
    // piece (K % 8), an M/N-major one's K is free
    if ((A && !aligned16(A)) || (B && !aligned16(B)) || !aligned16(Out) ||
        (beta != 0.0f && !aligned16(C)) || lda % 8 != 0 || ldb % 8 != 0 ||
        ((!a_mn || !b_mn) && K % 8 != 0))
        return TCM_ERR_MISALIGNED;
    DeviceInfo dev;
    if ((s = device_info(&dev)) != TCM_OK) return s;
    const int32_t chosen = choose_variant(1, M, N, 16, dev.cus);
    // the plain kernels read dense storage only (rows K and N apart)
    const bool plain_epi = alpha == 1.0f && beta == 0.0f && out_dtype != TCM_F16 && lda == K &&
                           ldb == K && ldo == N && op == TCM_OP_IDENTITY;
    int32_t v = (a_mn || b_mn) ? mn_variant(chosen)
                : plain_epi    ? chosen
                               : epi_variant(chosen);
    // the 128 x 64 tile has no LDS room for the per-element epilogue
    if (op != TCM_OP_IDENTITY && v == V_T128x64) v = V_T128x128;
    tcm_plan plan;
    GemmArgs a;
    plan_variant(v, 1, M, N, K, dev.cus, &plan, &a);
    a.A = A;
    a.B = B;
    a.C = Out;
    a.lda = (int32_t)lda;
    a.ldb = (int32_t)ldb;
    a.ldc = (int32_t)ldo;
    a.Cin = beta != 0.0f ? C : nullptr;
    a.ldcin = beta != 0.0f ? (int32_t)ldc : 0;
    a.alpha = alpha;
    a.beta = beta;
    a.c_dtype = (int32_t)c_dtype;
    a.op = (int32_t)op;
    hipError_t e;
    const hipStream_t st = (hipStream_t)stream;
    if (a_mn && b_mn)
        e = launch_gemm_mn<true, true>(v, (int32_t)dtype, (int32_t)out_dtype, a, plan.grid, st);
    else if (a_mn)
        e = launch_gemm_mn<true, false>(v, (int32_t)dtype, (int32_t)out_dtype, a, plan.grid, st);
    else if (b_mn)
        e = launch_gemm_mn<false, true>(v, (int32_t)dtype, (int32_t)out_dtype, a, plan.grid, st);
    else if (plain_epi)
        e = launch_gemm_tn(v, (int32_t)dtype, (int32_t)out_dtype, a, plan.grid, st);
    else
        e = launch_gemm_epi(v, (int32_t)dtype, (int32_t)out_dtype, a, plan.grid, st);
    return e == hipSuccess ? TCM_OK : TCM_ERR_HIP;
}

tcm_status tcm_plan_gemm(int64_t batch, int64_t M, int64_t N, int64_t K, tcm_dtype dtype,
                         tcm_dtype out_dtype, int mx, int num_cus, tcm_plan* plan) {
    if (!plan) return TCM_ERR_NULL_POINTER;
    if (mx < 0 || mx > 5) return TCM_ERR_INVALID_ARGUMENT;
    const bool out_ok = out_dtype == TCM_F32 || out_dtype == TCM_BF16 ||
                        (mx == 4 && out_dtype == TCM_F16);
    if (mx ? !out_ok : !plain_pair(dtype, out_dtype)) return TCM_ERR_UNSUPPORTED_DTYPE;
    bool empty = false;
    tcm_status s = check_sizes(batch, M, N, K, &empty);
    if (s != TCM_OK) return s;
    if ((s = check_range(batch, M, N, K)) != TCM_OK) return s;
    if (mx && K % 32 != 0) return TCM_ERR_UNSUPPORTED_SHAPE;
    if (num_cus <= 0) {
        DeviceInfo dev;
        if ((s = device_info(&dev)) != TCM_OK) return s;
        num_cus = dev.cus;
    }
    const int64_t b1 = batch < 1 ? 1 : batch, m1 = M < 1 ? 1 : M, n1 = N < 1 ? 1 : N;
    if (mx == 4)
        plan_variant(nv4_variant(m1, n1, K > 0 && K % 256 == 0, num_cus), b1, m1, n1, K, num_cus,
                     plan, nullptr);
    else if (mx == 5)
        // (dense storage: leading dimensions M and N rounded to 16, ldo = N)
        plan_variant(mx_mn_variant(m1, n1, K, (m1 + 15) / 16 * 16, (n1 + 15) / 16 * 16, n1, true,
                                   num_cus),
                     b1, m1, n1, K, num_cus, plan, nullptr);
    else if (mx == 3)
        // (word-aligned scale tensors)
        plan_variant(mx6_variant(choose_variant(b1, m1, n1, 6, num_cus), K > 0 && K % 128 == 0,
                                 K > 0 && K % 512 == 0),
                     b1, m1, n1, K, num_cus, plan, nullptr);
    else if (mx == 1)
        // (16-byte aligned scale tensors)
        plan_variant(mx8_variant(choose_variant(b1, m1, n1, 8, num_cus), K > 0 && K % 512 == 0),
                     b1, m1, n1, K, num_cus, plan, nullptr);
    else if (mx == 2)
        // (16-byte aligned scale tensors)
        plan_variant(mx4_variant(choose_variant(b1, m1, n1, 4, num_cus), K > 0 && K % 512 == 0),
                     b1, m1, n1, K, num_cus, plan, nullptr);
    else
        make_plan(b1, m1, n1, K, mx == 2 ? 4 : mx ? 8 : 16, num_cus, plan, nullptr);
    if (empty) {
        plan->grid = 0;
        plan->tiles = 0;
    }
    return TCM_OK;
}

const char* tcm_status_string(tcm_status s) {
    switch (s) {
    case TCM_OK: return "TCM_OK: success";
    case TCM_ERR_NULL_POINTER: return "TCM_ERR_NULL_POINTER: a required pointer is NULL";
    case TCM_ERR_INVALID_SHAPE: return "TCM_ERR_INVALID_SHAPE: negative size or size overflow";
    case TCM_ERR_UNSUPPORTED_SHAPE:
        return "TCM_ERR_UNSUPPORTED_SHAPE: size outside the supported range (K <= 2^20, M and N "
               "<= 2^30, MX K a multiple of 32)";
    case TCM_ERR_MISALIGNED:
        return "TCM_ERR_MISALIGNED: pointers and operand rows must be 16-byte aligned";
    case TCM_ERR_UNSUPPORTED_DTYPE: return "TCM_ERR_UNSUPPORTED_DTYPE: dtype pair not supported";
    case TCM_ERR_NO_DEVICE: return "TCM_ERR_NO_DEVICE: no gfx950 HIP device is current";
    case TCM_ERR_HIP: return "TCM_ERR_HIP: a HIP runtime call or kernel launch failed";
    case TCM_ERR_INVALID_ARGUMENT:
        return "TCM_ERR_INVALID_ARGUMENT: an order or operation code outside its values";
    }
    return "TCM_ERR_UNKNOWN: unknown status code";
}

}  // extern "C"
