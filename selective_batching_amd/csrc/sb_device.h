// Device-side declarations shared by the kernel translation units of libsb.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sb_internal.h"

namespace sb {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16, round to nearest, ties to even (NaN stays NaN)
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int DT> struct Store;
template <> struct Store<SB_F32> {
    using T = float;
    __device__ static float ld(const float* p) { return *p; }
    __device__ static void st(float* p, float v) { *p = v; }
};
template <> struct Store<SB_BF16> {
    using T = uint16_t;
    __device__ static float ld(const uint16_t* p) { return bf2f(*p); }
    __device__ static void st(uint16_t* p, float v) { *p = f2bf(v); }
};

// Workgroup index remap so that consecutive logical tiles run on the same XCD
// (workgroups are dealt to the 8 XCDs round-robin by hardware).
__device__ __forceinline__ int xcd_remap(int pid, int total) {
    const int per = total / 8, rem = total % 8;
    const int x = pid % 8, local = pid / 8;
    return x * per + (x < rem ? x : rem) + local;
}

// ------------------------------------------------------------------ global -> LDS copies
typedef __attribute__((address_space(3))) void lds_void;

// vmcnt <= n (other counters untouched): gfx9 encoding, vmcnt in bits 3:0 and 15:14
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One 16-byte-per-lane global -> LDS transfer (global_load_lds_dwordx4): lane i
// of the wave writes LDS bytes [lds_base + 16 i, +16).  Issued from inline
// assembly so that the compiler's wait insertion does not see it: the caller
// orders it with its own vmcnt waits and barriers.  lds_base is wave-uniform.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}

// Workgroup barrier that is also a compiler memory barrier (no LDS access moves across it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_void*)p; }

// ------------------------------------------------------------------ GEMM
enum { EPI_STORE = 0, EPI_GELU = 1, EPI_RESID = 2, EPI_SWIGLU = 3 };

struct GemmArgs {
    int M, N, K;            // output [M, N]; for SWIGLU N = F (W has 2F rows: gate then up)
    const void* A;          // [M, K] (dtype), row stride lda
    long long lda;
    const void* W;          // [N or 2F, K] (dtype), row stride ldw
    long long ldw;
    const void* bias;       // [N] (dtype) or NULL
    void* C;                // output (dtype, or fp32 if out_f32); for RESID: fp32 x, updated in place
    long long ldc;
    int out_f32;
    int F;                  // SwiGLU: offset of the up rows in W
};

int launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s);
// Compute units of the current device (256 on MI355X; 256 if the query fails).
int num_cus();

// ------------------------------------------------------------------ timing hooks
void timing_begin(int kind, hipStream_t s);
void timing_end(int kind, hipStream_t s);

struct TimedScope {
    int k;
    hipStream_t s;
    TimedScope(int kind, hipStream_t st) : k(kind), s(st) { timing_begin(k, s); }
    ~TimedScope() { timing_end(k, s); }
};

int check_launch(const char* what);

}  // namespace sb
