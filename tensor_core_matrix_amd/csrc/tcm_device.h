// Device-side building blocks of the gfx950 (CDNA4) tiled product kernels:
// buffer resources, direct global->LDS copies, explicit wait counters and the
// MFMA / epilogue primitives.
#pragma once

#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "tcm_internal.h"

namespace tcm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaveSize = 64;
// A buffer offset that is past every buffer's num_records: buffer loads at it
// return zeros (used for the K tail).
constexpr uint32_t kOutOfRange = 0x80000000u;

#define TCM_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Raw buffer resource over `bytes` bytes at `base`; loads past `bytes` give 0.
// Word 3 = 0x00020000 selects a 32-bit data format, which untyped loads need
// to return data at all on gfx9-family parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes per lane from the buffer straight into LDS, bypassing VGPRs.  The
// 64 lanes of the wave fill 1 KiB of LDS contiguously from `lds_wave_base`
// (lane l writes bytes [16 l, 16 l + 16)); only the global side is gathered.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds_wave_base,
                                              uint32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, TCM_LDS_PTR(lds_wave_base), 16, voffset, 0, 0, 0);
}

// The same 16-byte copy written as inline assembly, for kernels that read LDS
// with transposing reads.  After a copy issued through the builtin, the
// compiler waits for every copy in flight (vmcnt(0)) before each transposing
// read, which it cannot tell apart from the copy's destination; that wait
// would drain the copy pipeline at every fragment read.  Kernels order their
// copies and reads with explicit vmcnt waits and a barrier before a stage is
// read, so the assembly form changes no ordering they rely on.  M0 (the LDS
// destination) is an input, so the compiler sets it; one wait state after
// the M0 write precedes the copy, which reads M0.
__device__ __forceinline__ void copy16_to_lds_asm(__amdgpu_buffer_rsrc_t r, void* lds_wave_base,
                                                  uint32_t voffset) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base;
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(r), "{m0}"(m0)
                 : "memory");
}

// 4 bytes per lane from the buffer into LDS: the wave fills 256 bytes
// contiguously from `lds_wave_base` (lane l writes bytes [4 l, 4 l + 4)).
__device__ __forceinline__ void copy4_to_lds(__amdgpu_buffer_rsrc_t r, void* lds_wave_base,
                                             uint32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, TCM_LDS_PTR(lds_wave_base), 4, voffset, 0, 0, 0);
}

// The 4-byte copy as inline assembly, for the same kernels as
// copy16_to_lds_asm.
__device__ __forceinline__ void copy4_to_lds_asm(__amdgpu_buffer_rsrc_t r, void* lds_wave_base,
                                                 uint32_t voffset) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base;
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(r), "{m0}"(m0)
                 : "memory");
}

// Transposing 8-byte LDS read of 16-bit elements (ds_read_b64_tr_b16).  The
// lanes act in groups of 16; within a group, lane t addresses 8 bytes (4
// elements), the group's 16 addresses forming a 4 x 16 block whose row r is
// what lanes 4 r .. 4 r + 3 address, in lane order.  Lane t receives column t
// of that block: element t of each of the 4 rows.  (Established on the device
// by reading an LDS array that holds each element's own index.)
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4_t lds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p));
}

// ds_read_b64_tr_b8: lane t of each 16-lane group receives byte t of the 8
// rows of 16 bytes its group addresses (row r from lanes 2r, 2r + 1).
__device__ __forceinline__ i32x2_t lds_read_tr8(const void* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2_t*)(p));
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier after this wave's LDS reads have returned.  Unlike
// __syncthreads() it does not wait for outstanding global loads, so the
// copies of later stages stay in flight across it.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Lanes of one wave exchanging data through LDS.  The hardware runs a wave's
// LDS operations in issue order, so no wait is needed between a lane's write
// and another lane's read; but the compiler reasons lane by lane and may move
// or forward a load across such a write (it sank the read-back of a staging
// area into a branch taken by only the writing lanes).  This compiler-only
// fence keeps every memory access on its side.
__device__ __forceinline__ void wave_lds_exchange() { asm volatile("" ::: "memory"); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

template <typename TOut>
__device__ __forceinline__ TOut convert_out(float x);
template <>
__device__ __forceinline__ float convert_out<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 convert_out<__bf16>(float x) { return to_bf16(x); }
// fp32 -> fp16, round to nearest even (v_cvt_f16_f32); beyond the range: inf
template <>
__device__ __forceinline__ _Float16 convert_out<_Float16>(float x) { return (_Float16)x; }

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Four consecutive outputs of one row (8 bytes bf16 / 16 bytes fp32).
template <typename TOut>
__device__ __forceinline__ void store4(TOut* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
    *(f32x4_t*)dst = (f32x4_t){a, b, c, d};
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* dst, float a, float b, float c, float d) {
    *(bf16x4_t*)dst = (bf16x4_t){to_bf16(a), to_bf16(b), to_bf16(c), to_bf16(d)};
}
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* dst, float a, float b, float c, float d) {
    *(f16x4_t*)dst = (f16x4_t){(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
}

// f(std::integral_constant<int, 0>{}) .. f(std::integral_constant<int, N-1>{})
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// 16 bytes of accumulator values into LDS, written from accumulation
// registers (ds_write_b128 with an AGPR source) by inline assembly.  The
// builtin store form first copies the values to VGPRs; in the epilogue with a
// per-element operation, whose loop keeps all 256 accumulators of a lane
// live, those copies made the register allocator spill accumulators.  LDS
// operations of a wave complete in order, so a later read of the same bytes
// by any lane of the wave sees them; the compiler's own lgkmcnt waits are
// only made longer by the extra operation.
__device__ __forceinline__ void lds_write16_acc(void* lds_dst, f32x4_t v) {
    const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_dst;
    asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "a"(v) : "memory");
}

// Per-element epilogue operations, codes of tcm_op: applied in fp32 to the
// finished value alpha * sum + beta * c, before the rounding to the output
// type.  The exponential and reciprocal are the hardware's base-2
// exponential (v_exp_f32) and reciprocal (v_rcp_f32), about 1 ulp each.
enum : int { kOpIdentity = 0, kOpRelu = 1, kOpGeluTanh = 2, kOpGeluErf = 3, kOpSilu = 4 };
constexpr int kNumOps = 5;

// 1 / (1 + e^-y); 0 for large negative y (e^-y overflows to inf)
__device__ __forceinline__ float logistic(float y) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y * 1.4426950408889634f));
}

template <int OP>
__device__ __forceinline__ float apply_op(float x) {
    if constexpr (OP == kOpRelu) {
        return x > 0.0f ? x : 0.0f;
    } else if constexpr (OP == kOpSilu) {
        return x * logistic(x);
    } else if constexpr (OP == kOpGeluTanh) {
        // x/2 (1 + tanh u) = x logistic(2u), u = sqrt(2/pi) (x + 0.044715 x^3)
        const float u = 0.7978845608028654f * (x + 0.044715f * x * x * x);
        return x * logistic(2.0f * u);
    } else if constexpr (OP == kOpGeluErf) {
        // x Phi(x) = x/2 erfc(-x/sqrt 2).  erfc(z) for z >= 0 from Abramowitz
        // and Stegun, Handbook of Mathematical Functions, 7.1.26:
        // t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-z^2), t = 1 / (1 + p z),
        // absolute error at most 1.5e-7.  Negative x uses erfc(-z) = 2 - erfc(z).
        const float z = fabsf(x) * 0.7071067811865476f;
        const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * z);
        const float poly =
            t * (0.254829592f +
                 t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
        const float q = poly * __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);  // erfc(z)
        return x >= 0.0f ? x * (1.0f - 0.5f * q) : 0.5f * x * q;
    } else {
        return x;
    }
}

// Values of a C input as floats; dt is the tcm_dtype code (0 f16, 1 bf16,
// 2 f32).  load4_c reads elements n .. n+3 of a row in one access (n a
// multiple of 4, the row start aligned to 4 elements).
__device__ __forceinline__ f32x4_t load4_c(const char* row, int n, int dt) {
    if (dt == 2) return *(const f32x4_t*)(row + 4 * (int64_t)n);
    if (dt == 1) {
        const bf16x4_t v = *(const bf16x4_t*)(row + 2 * (int64_t)n);
        return (f32x4_t){(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
    const f16x4_t v = *(const f16x4_t*)(row + 2 * (int64_t)n);
    return (f32x4_t){(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ float load1_c(const char* row, int n, int dt) {
    if (dt == 2) return ((const float*)row)[n];
    if (dt == 1) return (float)((const __bf16*)row)[n];
    return (float)((const _Float16*)row)[n];
}

// XCD-aware workgroup order.  Workgroups are dealt round-robin to the 8 XCDs
// (workgroup b runs on XCD b % 8), each with its own L2.  Renumbering so that
// the G/8 workgroups of one XCD take consecutive logical ids makes them work on
// neighbouring output tiles, which share A rows and B rows in that L2.
__device__ __forceinline__ int logical_block(int b, int G) {
    if (G % 8 != 0) return b;
    return (b % 8) * (G / 8) + b / 8;
}

// Grouped tile order: tiles advance down `group_m` tile rows before moving to
// the next tile column, so concurrently running tiles share operand rows.
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int t, int& batch, int& tm,
                                            int& tn) {
    batch = t / p.tiles_per_batch;
    int r = t - batch * p.tiles_per_batch;
    int gsz = p.group_m * p.tiles_n;
    int grp = r / gsz;
    int first = grp * p.group_m;
    int gm = min(p.group_m, p.tiles_m - first);
    int rr = r - grp * gsz;
    tm = first + rr % gm;
    tn = rr / gm;
}

}  // namespace tcm
