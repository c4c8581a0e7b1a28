// Token-wise linear layers over the flattened [T, K] activation: C = A W^T.
//
// Selective batching runs every non-attention operator on the [sum L_i, H]
// tensor so that each weight is read once per iteration for all requests
// ("连续批处理完全拆解", section 观察; "CS349D Lecture 2", section 4.2).  T is
// arbitrary (ragged), so rows beyond T are masked; N and K come from the model.
//
// bf16: v_mfma_f32_16x16x32_bf16 tiles.  Large GEMMs: 256 x 256 (or 256 x 192,
// 192 x 256, 256 x 384, 224 x 384) workgroup tiles of 8 waves, two waves per
// SIMD, two LDS stages of 64-deep K filled straight from global memory
// (global_load_lds, XOR-swizzled rows: no bank conflicts on the operand reads),
// XCD-aware grouped tile order, the shape picked per GEMM from the rounds of
// tiles over the CUs.  Small GEMMs (decode-heavy batches): register-ring tiles
// of 32 to 128 rows (K steps of loads in flight in registers, loading-only
// waves beside the computing ones), by a per-CU bytes cost model.
// fp32: 16x16x4 fp32 MFMA tiles with a fixed, ascending K order.
// Epilogues fuse bias, exact GeLU, SwiGLU (SiLU(gate) * up) or the residual
// add into the fp32 stream x.
#include <algorithm>
#include <cstdlib>

#include "sb_device.h"

namespace sb {
namespace {

__device__ __forceinline__ float gelu_exact(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

template <int DT>
__device__ __forceinline__ float bias_at(const void* b, int n) {
    return b ? Store<DT>::ld((const typename Store<DT>::T*)b + n) : 0.0f;
}

// Store one finished output value (non-SwiGLU epilogues).
template <int DT, int EPI>
__device__ __forceinline__ void epi_store(const GemmArgs& a, int m, int n, float acc) {
    float v = acc + bias_at<DT>(a.bias, n);
    if (EPI == EPI_GELU) v = gelu_exact(v);
    if (EPI == EPI_RESID) {
        float* x = (float*)a.C + (long long)m * a.ldc + n;
        *x = *x + v;
    } else if (a.out_f32) {
        ((float*)a.C)[(long long)m * a.ldc + n] = v;
    } else {
        Store<DT>::st((typename Store<DT>::T*)a.C + (long long)m * a.ldc + n, v);
    }
}

template <int DT>
__device__ __forceinline__ void swiglu_store(const GemmArgs& a, int m, int f, float g, float u) {
    float v = silu(g) * u;
    if (a.out_f32)
        ((float*)a.C)[(long long)m * a.ldc + f] = v;
    else
        Store<DT>::st((typename Store<DT>::T*)a.C + (long long)m * a.ldc + f, v);
}

// Four consecutive outputs of one row as one 16-byte (fp32) or 8-byte (bf16) access.
__device__ __forceinline__ void store4(const GemmArgs& a, long long off, const f32x4& v) {
    if (a.out_f32) {
        *(f32x4*)((float*)a.C + off) = v;
    } else {
        const uint32_t lo = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        const uint32_t hi = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
        *(u32x2*)((uint16_t*)a.C + off) = u32x2{lo, hi};
    }
}

// Whether outputs n..n+3 of a row may be written as one vector access: ldc and the
// base pointer aligned for it (checked once per launch, wave-uniform).
__device__ __forceinline__ bool vec4_ok(const GemmArgs& a, int epi) {
    const int align = (epi == EPI_RESID || a.out_f32) ? 16 : 8;
    return (a.ldc & 3) == 0 && ((uintptr_t)a.C & (uintptr_t)(align - 1)) == 0;
}

// Epilogue of outputs (m, n..n+3): v[r] is the accumulator of column n + r.
template <int EPI>
__device__ __forceinline__ void epi_store4(const GemmArgs& a, bool vec, int m, int n, f32x4 v) {
    if (m >= a.M) return;
    if (vec && n + 3 < a.N) {
        if (a.bias) {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] += bias_at<SB_BF16>(a.bias, n + r);
        }
        if (EPI == EPI_GELU) {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = gelu_exact(v[r]);
        }
        const long long off = (long long)m * a.ldc + n;
        if (EPI == EPI_RESID) {
            f32x4* x = (f32x4*)((float*)a.C + off);
            *x = *x + v;
        } else {
            store4(a, off, v);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (n + r < a.N) epi_store<SB_BF16, EPI>(a, m, n + r, v[r]);
    }
}

// SwiGLU outputs (m, f..f+3) from gate accumulators g and up accumulators u.
__device__ __forceinline__ void swiglu_store4(const GemmArgs& a, bool vec, int m, int f, const f32x4& g,
                                              const f32x4& u) {
    if (m >= a.M) return;
    if (vec && f + 3 < a.N) {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = silu(g[r]) * u[r];
        store4(a, (long long)m * a.ldc + f, v);
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (f + r < a.N) swiglu_store<SB_BF16>(a, m, f + r, g[r], u[r]);
    }
}

// Epilogue of one wave's MI x NI blocks of C^T = W A^T.  The MFMAs take the
// W fragment as their first operand, so lane (lr = lane % 16, lc = lane / 16)
// of block (i, j) holds row m_lane + 16 i and the four consecutive columns
// n_lane + 16 j + {0..3}: rows are written as 16- or 8-byte pieces.  For
// SwiGLU the wave's blocks j < NI/2 are gate columns and j + NI/2 the matching
// up columns; n_lane then indexes the output (F) columns.
template <int MI, int NI, int EPI>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& a, const f32x4 (&acc)[MI][NI], int m_lane, int n_lane) {
    const bool vec = vec4_ok(a, EPI);
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI / 2; ++j)
                swiglu_store4(a, vec, m_lane + 16 * i, n_lane + 16 * j, acc[i][j], acc[i][j + NI / 2]);
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) epi_store4<EPI>(a, vec, m_lane + 16 * i, n_lane + 16 * j, acc[i][j]);
    }
}

// ================================================================== bf16 MFMA
// Workgroup tile BM x BN (BN counts W rows; for SwiGLU each wave's WN rows
// are WN/2 gate rows then the matching WN/2 up rows), WAVES_M x WAVES_N waves,
// wave tile WM x WN of 16 x 16 MFMA blocks, K in steps of 64 through two LDS
// stages.  Each output element is one MFMA chain over K in ascending 32-wide
// steps, whatever the tile shape: results do not depend on M or on the tile a
// row falls in.
template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_bf16_kernel(GemmArgs a) {
    constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    constexpr int BK = 64, LDSK = BK + 8;            // 144-byte rows: conflict-free 16-byte reads
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int MI = WM / 16, NI = WN / 16;
    constexpr int CH = BK / 8;                       // 16-byte chunks per row
    constexpr int A_CH = BM * CH / THREADS, B_CH = BN * CH / THREADS;
    static_assert(A_CH * THREADS == BM * CH && B_CH * THREADS == BN * CH, "tile / thread mismatch");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDSK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDSK];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int out_cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int tiles_n = (a.N + out_cols - 1) / out_cols;
    const int total = tiles_m * tiles_n;
    const int pid = xcd_remap(blockIdx.x, total);
    // grouped order: GROUP_M row tiles sweep the column tiles together (L2 reuse of both operands)
    constexpr int GROUP_M = 4;
    const int per_group = GROUP_M * tiles_n;
    const int grp = pid / per_group;
    const int first_m = grp * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (pid % per_group) % gsz;
    const int tn = (pid % per_group) / gsz;
    const int m0 = tm * BM;

    const uint16_t* A = (const uint16_t*)a.A;
    const uint16_t* W = (const uint16_t*)a.W;

    // global row of every chunk this thread moves (clamped: rows past the end are loaded but never stored)
    const uint16_t* pa[A_CH];
    const uint16_t* pb[B_CH];
#pragma unroll
    for (int q = 0; q < A_CH; ++q) {
        const int c = tid + THREADS * q, row = c / CH, kc = (c % CH) * 8;
        pa[q] = A + (long long)min(m0 + row, a.M - 1) * a.lda + kc;
    }
#pragma unroll
    for (int q = 0; q < B_CH; ++q) {
        const int c = tid + THREADS * q, row = c / CH, kc = (c % CH) * 8;
        int gr;
        if (EPI == EPI_SWIGLU) {
            const int w = row / WN, cc = row % WN;
            const int f = tn * (BN / 2) + w * (WN / 2) + (cc % (WN / 2));
            gr = min(f, a.N - 1) + (cc >= WN / 2 ? a.F : 0);
        } else {
            gr = min(tn * BN + row, a.N - 1);
        }
        pb[q] = W + (long long)gr * a.ldw + kc;
    }

    u32x4 ra[A_CH], rb[B_CH];
    auto load = [&](int k0) {
#pragma unroll
        for (int q = 0; q < A_CH; ++q) ra[q] = *(const u32x4*)(pa[q] + k0);
#pragma unroll
        for (int q = 0; q < B_CH; ++q) rb[q] = *(const u32x4*)(pb[q] + k0);
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int q = 0; q < A_CH; ++q) {
            const int c = tid + THREADS * q;
            *(u32x4*)&As[buf][(c / CH) * LDSK + (c % CH) * 8] = ra[q];
        }
#pragma unroll
        for (int q = 0; q < B_CH; ++q) {
            const int c = tid + THREADS * q;
            *(u32x4*)&Bs[buf][(c / CH) * LDSK + (c % CH) * 8] = rb[q];
        }
    };

    f32x4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = a.K / BK;
    load(0);
    stash(0);
    __syncthreads();
    const int lrow = lane & 15, lk = (lane >> 4) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 bfr[NI];
#pragma unroll
            for (int j = 0; j < NI; ++j)
                bfr[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)&Bs[buf][(wn * WN + j * 16 + lrow) * LDSK + ks * 32 + lk]);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const bf16x8 af = __builtin_bit_cast(bf16x8, *(const u32x4*)&As[buf][(wm * WM + i * 16 + lrow) * LDSK + ks * 32 + lk]);
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af, acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) stash(buf ^ 1);
        __syncthreads();
    }

    const int n_lane = (EPI == EPI_SWIGLU ? tn * (BN / 2) + wn * (WN / 2) : tn * BN + wn * WN) + (lane >> 4) * 4;
    tile_epilogue<MI, NI, EPI>(a, acc, m0 + wm * WM + lrow, n_lane);
}

// ================================================================== bf16 MFMA, register ring
// Small problems (decode-heavy batches): few workgroups, each walking all of K.
// Loads go to registers first -- a ring of PF BK-deep K tiles per thread, each
// load issued PF steps before its tile is used -- and each tile is copied to LDS
// (two buffers, padded rows) one step before its MFMAs.  A step costs a fixed
// latency (copy to LDS, barrier, operand reads, MFMA chain) besides its bytes, so
// deeper steps move more bytes per step: 128-deep steps with 4 in flight take the
// 8B-shaped FFN2 at 64 rows from 46 to 37 us against 64-deep steps with 8 in
// flight (same bytes in flight).  With LW = 2 or 4 the workgroup has that many
// times the waves its MFMAs need: all of them load and copy, the first NCW
// compute, so the CU keeps more loads outstanding (64 x 64 tiles at 330 rows:
// QKV 55 -> 44 us; 32 x 32 tiles with 256-deep steps and LW = 4 at 64 rows:
// attention-out 12.0 -> 10.0 us).
// Same operand layout, MFMA and K order (32-wide MFMA steps, ascending) as
// gemm_bf16_kernel, so results are bitwise those of every other configuration.
template <int BM, int BN, int WAVES_M, int WAVES_N, int PF, int EPI, int BK, int LW>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N * LW) void gemm_bf16_ring_kernel(GemmArgs a) {
    static_assert(PF % 2 == 0, "ring slot parity selects the LDS buffer");
    static_assert(BK % 64 == 0, "K depth of a step");
    constexpr int THREADS = 64 * WAVES_M * WAVES_N * LW;
    constexpr int NCW = WAVES_M * WAVES_N;           // waves that compute; all LW x NCW waves load
    constexpr int LDSK = BK + 8;                     // rows padded by 16 bytes: conflict-free 16-byte reads
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int MI = WM / 16, NI = WN / 16;
    constexpr int CH = BK / 8;                       // 16-byte chunks per row
    constexpr int A_CH = BM * CH / THREADS, B_CH = BN * CH / THREADS;
    static_assert(A_CH * THREADS == BM * CH && B_CH * THREADS == BN * CH, "tile / thread mismatch");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDSK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDSK];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = (wave % NCW) / WAVES_N, wn = (wave % NCW) % WAVES_N;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int out_cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int tiles_n = (a.N + out_cols - 1) / out_cols;
    const int pid = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tm = pid % tiles_m, tn = pid / tiles_m;     // row tiles of one column block: same XCD
    const int m0 = tm * BM;

    const uint16_t* A = (const uint16_t*)a.A;
    const uint16_t* W = (const uint16_t*)a.W;
    // global row of every chunk this thread moves (clamped: rows past the end are loaded but never stored);
    // consecutive threads take consecutive 16-byte chunks, so one load instruction reads whole lines
    const uint16_t* pa[A_CH];
    const uint16_t* pb[B_CH];
#pragma unroll
    for (int q = 0; q < A_CH; ++q) {
        const int c = tid + THREADS * q, row = c / CH, kc = (c % CH) * 8;
        pa[q] = A + (long long)min(m0 + row, a.M - 1) * a.lda + kc;
    }
#pragma unroll
    for (int q = 0; q < B_CH; ++q) {
        const int c = tid + THREADS * q, row = c / CH, kc = (c % CH) * 8;
        int gr;
        if (EPI == EPI_SWIGLU) {
            const int w = row / WN, cc = row % WN;
            const int f = tn * (BN / 2) + w * (WN / 2) + (cc % (WN / 2));
            gr = min(f, a.N - 1) + (cc >= WN / 2 ? a.F : 0);
        } else {
            gr = min(tn * BN + row, a.N - 1);
        }
        pb[q] = W + (long long)gr * a.ldw + kc;
    }

    const int nk = a.K / BK;
    u32x4 ra[PF][A_CH], rb[PF][B_CH];
    auto load = [&](int s, int kt) {                 // ring slot s <- K tile kt (clamped to the last)
        const int k0 = min(kt, nk - 1) * BK;
#pragma unroll
        for (int q = 0; q < A_CH; ++q) ra[s][q] = *(const u32x4*)(pa[q] + k0);
#pragma unroll
        for (int q = 0; q < B_CH; ++q) rb[s][q] = *(const u32x4*)(pb[q] + k0);
    };
    auto stash = [&](int s, int buf) {
#pragma unroll
        for (int q = 0; q < A_CH; ++q) {
            const int c = tid + THREADS * q;
            *(u32x4*)&As[buf][(c / CH) * LDSK + (c % CH) * 8] = ra[s][q];
        }
#pragma unroll
        for (int q = 0; q < B_CH; ++q) {
            const int c = tid + THREADS * q;
            *(u32x4*)&Bs[buf][(c / CH) * LDSK + (c % CH) * 8] = rb[s][q];
        }
    };

    f32x4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int lrow = lane & 15, lk = (lane >> 4) * 8;
    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 bfr[NI];
#pragma unroll
            for (int j = 0; j < NI; ++j)
                bfr[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)&Bs[buf][(wn * WN + j * 16 + lrow) * LDSK + ks * 32 + lk]);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const bf16x8 af = __builtin_bit_cast(bf16x8, *(const u32x4*)&As[buf][(wm * WM + i * 16 + lrow) * LDSK + ks * 32 + lk]);
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af, acc[i][j], 0, 0, 0);
            }
        }
    };

    // loads go out in ring order, in the prologue and in the loop, so that before each step
    // only that step's loads have to be waited for
#pragma unroll
    for (int s = 0; s < PF; ++s) {
        load(s, s);
        __builtin_amdgcn_sched_barrier(0);
    }
    // step kt: copy ring slot kt % PF to LDS buffer kt & 1 (read last by step kt - 2, which every
    // wave finished before the barrier of step kt - 1), barrier, refill the slot with tile
    // kt + PF, MFMAs of buffer kt & 1.  Only the MFMAs depend on kt < nk: the copies and loads of
    // the steps past the end (at most PF - 1, of the clamped last tile) keep one fixed load order
    // on every path, which is what lets the waits stay PF - 1 steps deep across the loop.
    for (int kt0 = 0; kt0 < nk; kt0 += PF) {
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            stash(s, s & 1);
            __syncthreads();
            load(s, kt0 + s + PF);
            if (kt0 + s < nk && wave < NCW) compute(s & 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (wave >= NCW) return;                         // a loading-only wave

    const int n_lane = (EPI == EPI_SWIGLU ? tn * (BN / 2) + wn * (WN / 2) : tn * BN + wn * WN) + (lane >> 4) * 4;
    tile_epilogue<MI, NI, EPI>(a, acc, m0 + wm * WM + lrow, n_lane);
}

// ================================================================== bf16 MFMA, DMA-fed
// BM x BN tile, K in steps of BK (32 or 64) through a ring of STAGES LDS
// stages filled by global_load_lds_dwordx4 (16 bytes per lane from global
// memory straight into LDS, no staging registers).  A stage holds the A tile
// then the B tile, each row-major [rows][BK]; row r keeps its BK/8 16-byte
// k-chunks in slots permuted by sw(r) = (r >> 1) % (BK/8), so the MFMA
// operand reads (16 rows x one chunk per lane group, 8 lanes per LDS pass)
// hit 8 different 16-byte bank groups.  One copy instruction fills 1 KB: 64/(BK/8)
// consecutive rows, each row's BK*2 bytes read as one contiguous run (a whole
// 128-byte line when BK = 64).  Step kt: wait for this wave's copies of tile kt,
// barrier (every wave's copies landed, every wave finished tile kt-1), issue
// tile kt+STAGES-1 into the stage tile kt-1 used, then the MFMAs of tile kt.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int STAGES_>
struct DmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
    static constexpr int NWAVES = WAVES_M * WAVES_N, THREADS = 64 * NWAVES;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, MI = WM / 16, NI = WN / 16;
    static constexpr int CH = BK / 8;                            // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;                          // rows per copy instruction
    static constexpr int STAGE_ELEMS = (BM + BN) * BK;           // A rows then B rows
    static constexpr int NA = BM / RPI, NCOPY = (BM + BN) / RPI; // copy instructions per stage, A's first
    // Copy order.  Contiguous: each wave issues A_INSTR copies of A and B_INSTR of W per stage (row blocks
    // wave * A_INSTR .., wave * B_INSTR ..).  Strided: copy c of a stage is issued by wave c % NWAVES, so a
    // wave issues PER or PER - 1.  The 224x384 tile needs the strided order (76 copies over 8 waves); for
    // the 256x384 tile it measured 2-4% faster (QKV and the GPT-175B-shaped GEMMs), for 256x256 1-3% slower.
    static constexpr bool EVEN = NA % NWAVES == 0 && (NCOPY - NA) % NWAVES == 0;
    static constexpr bool STRIDED = !EVEN || BN >= 384;
    static constexpr int A_INSTR = NA / NWAVES, B_INSTR = (NCOPY - NA) / NWAVES;
    static constexpr int PER = STRIDED ? (NCOPY + NWAVES - 1) / NWAVES : A_INSTR + B_INSTR;
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(NA * RPI == BM && NCOPY * RPI == BM + BN, "whole copy instructions per operand");
    // the two-stage ring waits for every copy before each step, so waves may issue different counts
    static_assert(!STRIDED || STAGES == 2, "the strided copy order needs two stages");
    static_assert(STAGES >= 2 && (STAGES - 2) * PER <= 63, "vmcnt range");
    static_assert(STAGES * STAGE_ELEMS * 2 <= 160 * 1024, "LDS");
};

// MINW waves per SIMD at least: 2 lets two 4-wave workgroups (or one 8-wave
// one) share a CU, so one wave's MFMAs fill the other's barrier and LDS waits.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int STAGES_, int MINW, int FEED, int EPI>
__global__ __launch_bounds__(64 * WAVES_M_ * WAVES_N_, MINW) void gemm_bf16_dma_kernel(GemmArgs a) {
    using C = DmaCfg<BM_, BN_, WAVES_M_, WAVES_N_, BK_, STAGES_>;
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, WAVES_N = C::WAVES_N, STAGES = C::STAGES;
    constexpr int WM = C::WM, WN = C::WN, MI = C::MI, NI = C::NI, CH = C::CH, RPI = C::RPI;
    constexpr int STAGE_ELEMS = C::STAGE_ELEMS, A_INSTR = C::A_INSTR, B_INSTR = C::B_INSTR, PER = C::PER;
    constexpr int NA = C::NA, NCOPY = C::NCOPY, NWAVES = C::NWAVES;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[STAGES * STAGE_ELEMS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int out_cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int tiles_n = (a.N + out_cols - 1) / out_cols;
    const int total = tiles_m * tiles_n;
    const int pid = xcd_remap(blockIdx.x, total);
    constexpr int GROUP_M = 4;
    const int per_group = GROUP_M * tiles_n;
    const int grp = pid / per_group;
    const int first_m = grp * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (pid % per_group) % gsz;
    const int tn = (pid % per_group) / gsz;
    const int m0 = tm * BM;

    const uint16_t* A = (const uint16_t*)a.A;
    const uint16_t* W = (const uint16_t*)a.W;
    // Copy instruction c of a stage (c < NCOPY) fills stage bytes [1024 c, 1024 (c + 1)): row block c
    // (rows RPI c ..) of A for c < NA, else row block c - NA of W.  Element offsets (32-bit: every
    // operand here is < 2^31 elements) of this lane's source chunk for a tile row: lane -> row lane / CH
    // of the instruction's rows, LDS slot lane % CH, source chunk slot ^ sw(row).
    auto a_src = [&](int row) {
        const int chunk = (lane % CH) ^ ((row >> 1) % CH);
        return min(m0 + row, a.M - 1) * (int)a.lda + chunk * 8;
    };
    auto b_src = [&](int row) {
        const int chunk = (lane % CH) ^ ((row >> 1) % CH);
        int gr;
        if (EPI == EPI_SWIGLU) {
            const int w = row / WN, cc = row % WN;
            const int f = tn * (BN / 2) + w * (WN / 2) + (cc % (WN / 2));
            gr = min(f, a.N - 1) + (cc >= WN / 2 ? a.F : 0);
        } else {
            gr = min(tn * BN + row, a.N - 1);
        }
        return gr * (int)a.ldw + chunk * 8;
    };
    int src[PER];
    uint32_t dstA = 0, dstB = 0;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    if constexpr (!C::STRIDED) {
        // the wave's copies are A blocks wave * A_INSTR .. and W blocks wave * B_INSTR ..
#pragma unroll
        for (int j = 0; j < A_INSTR; ++j) src[j] = a_src((wave * A_INSTR + j) * RPI + lane / CH);
#pragma unroll
        for (int j = 0; j < B_INSTR; ++j) src[A_INSTR + j] = b_src((wave * B_INSTR + j) * RPI + lane / CH);
        // LDS byte address of this wave's first A and B copy in stage 0 (wave-uniform, so scalar)
        dstA = __builtin_amdgcn_readfirstlane(lds_addr(smem) + wave * A_INSTR * 1024);
        dstB = __builtin_amdgcn_readfirstlane(lds_addr(smem) + BM * BK * 2 + wave * B_INSTR * 1024);
    } else {
        // the wave's copy d is the stage's copy wave + NWAVES d
#pragma unroll
        for (int d = 0; d < PER; ++d) {
            const int c = wv + NWAVES * d;
            src[d] = c < NA ? a_src(c * RPI + lane / CH) : b_src((c - NA) * RPI + lane / CH);
        }
        dstA = __builtin_amdgcn_readfirstlane(lds_addr(smem));
    }
    // copy instruction d of this wave (contiguous order: A copies first, then B) of the tile at k0 into `stage`
    auto piece = [&](int stage, int k0, int d) {
        const uint32_t so = (uint32_t)(stage * STAGE_ELEMS * 2);
        if constexpr (!C::STRIDED) {
            if (d < A_INSTR) dma16(A + (src[d] + k0), dstA + so + d * 1024);
            else dma16(W + (src[d] + k0), dstB + so + (d - A_INSTR) * 1024);
        } else {
            const int c = wv + NWAVES * d;           // wave-uniform
            if (c < NCOPY) dma16((c < NA ? A : W) + (src[d] + k0), dstA + so + c * 1024);
        }
    };
    auto issue = [&](int stage, int k0) {
#pragma unroll
        for (int d = 0; d < PER; ++d) piece(stage, k0, d);
    };

    f32x4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int lr = lane & 15, lc = lane >> 4;
    // element offset of this lane's operand (row lr of a 16-row block, chunk 4h + lc) for each 32-k half h
    int rd[BK / 32];
#pragma unroll
    for (int h = 0; h < BK / 32; ++h) rd[h] = lr * BK + (((4 * h + lc) ^ ((lr >> 1) % CH)) * 8);
    // MFMAs of the tile in `stage`, as G = (BK/32) * MI groups of NI MFMAs (one A fragment each).
    // FEED == 1: the copies of the next tile (into nstage, at nk0) go out one per group behind the
    // group's MFMAs, over the first PER groups, instead of all at once: a burst of copies from every
    // wave queues in the address unit and holds the waves back from their MFMAs.
    constexpr int G = (BK / 32) * MI;
    constexpr int PG = (PER + G - 1) / G;                  // copies per group
    auto spread_copies = [&](int g, int nstage, int nk0, bool more) {
#pragma unroll
        for (int q = 0; q < PG; ++q) {
            const int d = g * PG + q;
            if (d < PER && more) {
                __builtin_amdgcn_sched_barrier(0);
                piece(nstage, nk0, d);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    auto compute = [&](int stage, int nstage, int nk0, bool more) {
        const uint16_t* As = smem + stage * STAGE_ELEMS + (wm * WM) * BK;
        const uint16_t* Bs = smem + stage * STAGE_ELEMS + BM * BK + (wn * WN) * BK;
        auto ldA = [&](int h, int i) { return __builtin_bit_cast(bf16x8, *(const u32x4*)(As + i * 16 * BK + rd[h])); };
        auto ldB = [&](int h, int j) { return __builtin_bit_cast(bf16x8, *(const u32x4*)(Bs + j * 16 * BK + rd[h])); };
        {
#pragma unroll
            for (int h = 0; h < BK / 32; ++h) {
                bf16x8 bfr[NI];
#pragma unroll
                for (int j = 0; j < NI; ++j) bfr[j] = ldB(h, j);
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const bf16x8 af = ldA(h, i);
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af, acc[i][j], 0, 0, 0);
                    if constexpr (FEED == 1) spread_copies(h * MI + i, nstage, nk0, more);
                }
            }
        }
    };

    const int nk = a.K / BK;
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t)
        if (t < nk) issue(t, t * BK);
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
        // copies issued after tile kt that may stay in flight
        const int later = min(STAGES - 2, nk - 1 - kt);
        if (later == STAGES - 2) wait_vmcnt<(STAGES - 2) * PER>();
        else if (later == 0) wait_vmcnt<0>();
        else if (later == 1) wait_vmcnt<PER>();
        else if (later == 2) wait_vmcnt<2 * PER>();
        else wait_vmcnt<(3 * PER > 63 ? 63 : 3 * PER)>();
        lds_barrier();
        const int nstage = stage == 0 ? STAGES - 1 : stage - 1;
        const bool more = kt + STAGES - 1 < nk;
        if (FEED == 0 && more) issue(nstage, (kt + STAGES - 1) * BK);
        compute(stage, nstage, (kt + STAGES - 1) * BK, more);
        __builtin_amdgcn_sched_barrier(0);            // keep each tile's operands local to its step
        stage = (stage + 1 == STAGES) ? 0 : stage + 1;
    }

    const int n_lane = (EPI == EPI_SWIGLU ? tn * (BN / 2) + wn * (WN / 2) : tn * BN + wn * WN) + (lane >> 4) * 4;
    tile_epilogue<MI, NI, EPI>(a, acc, m0 + wm * WM + lr, n_lane);
}

// ================================================================== fp32 MFMA
// 64 x 64 tile (64 A rows x 64 W rows), 4 waves of 32 x 32 outputs (2 x 2 blocks of the 16x16x4 fp32
// MFMA), K in steps of 16 through LDS with the next step's global loads in flight in registers.  As in
// the bf16 kernels the W fragment is the MFMA's first operand, so lane (lr = lane % 16, g = lane / 16)
// of block (i, j) holds output row m0 + 16 i + lr and the four consecutive columns 16 j + 4 g + {0..3}.
// Each output is one MFMA chain over ascending K (4 at a time), whatever M and the tile a row falls in.
// SwiGLU: wave wn's 32 W rows are 16 gate rows and the matching 16 up rows, so block j = 0 holds gate
// and j = 1 up values of the same 16 output columns (a tile covers 32 output columns).
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_mfma_kernel(GemmArgs a) {
    constexpr int BK = 16, LDK = BK + 4;            // 80-byte rows: 16-byte aligned stores
    __shared__ __attribute__((aligned(16))) float As[2][64 * LDK];
    __shared__ __attribute__((aligned(16))) float Ws[2][64 * LDK];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1, lr = lane & 15, g = lane >> 4;
    const int out_cols = (EPI == EPI_SWIGLU) ? 32 : 64;
    const int tiles_n = (a.N + out_cols - 1) / out_cols;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * 64;
    const float* A = (const float*)a.A;
    const float* W = (const float*)a.W;
    // this thread copies 4 consecutive k of one A row and one W row per step
    const int cr = tid >> 2, ck = (tid & 3) * 4;
    const float* pa = A + (long long)min(m0 + cr, a.M - 1) * a.lda + ck;
    int wr;
    if (EPI == EPI_SWIGLU) {
        const int w = cr >> 5, cc = cr & 31;          // W tile row cr: wave w, gate (cc < 16) or up
        const int f = tn * 32 + w * 16 + (cc & 15);
        wr = min(f, a.N - 1) + (cc >= 16 ? a.F : 0);
    } else {
        wr = min(tn * 64 + cr, a.N - 1);
    }
    const float* pw = W + (long long)wr * a.ldw + ck;
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nk = a.K / BK;
    f32x4 ra = *(const f32x4*)pa, rw = *(const f32x4*)pw;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        *(f32x4*)&As[buf][cr * LDK + ck] = ra;
        *(f32x4*)&Ws[buf][cr * LDK + ck] = rw;
        __syncthreads();
        if (kt + 1 < nk) {
            ra = *(const f32x4*)(pa + (kt + 1) * BK);
            rw = *(const f32x4*)(pw + (kt + 1) * BK);
        }
#pragma unroll
        for (int kk = 0; kk < BK; kk += 4) {
            float av[2], wv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) av[i] = As[buf][(wm * 32 + i * 16 + lr) * LDK + kk + g];
#pragma unroll
            for (int j = 0; j < 2; ++j) wv[j] = Ws[buf][(wn * 32 + j * 16 + lr) * LDK + kk + g];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[j], av[i], acc[i][j], 0, 0, 0);
        }
        // the other buffer is written next step: every wave has finished reading it (it was read one
        // step ago, before this step's barrier)
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = m0 + wm * 32 + i * 16 + lr;
        if (m >= a.M) continue;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int f = tn * 32 + wn * 16 + 4 * g + r;
                if (f < a.N) swiglu_store<SB_F32>(a, m, f, acc[i][0][r], acc[i][1][r]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = tn * 64 + wn * 32 + j * 16 + 4 * g + r;
                    if (n < a.N) epi_store<SB_F32, EPI>(a, m, n, acc[i][j][r]);
                }
        }
    }
}

// Tile configurations of the bf16 kernel: {BM, BN, waves along M, waves along N}.
enum {
    CFG_128x128_4W = 0, CFG_256x256_4W, CFG_256x256_8W, CFG_256x128_4W, CFG_128x256_4W,   // register-staged
    CFG_DMA_256x256_8W_S4, CFG_DMA_256x128_4W_S3, CFG_DMA_128x256_4W_S3, CFG_DMA_256x256_8W_S5,  // DMA-fed, BK 32
    CFG_DMA_256x256_8W_K64_S2, CFG_DMA_256x256_4W_K64_S2,                                     // DMA-fed, BK 64
    CFG_DMA_256x256_8W_K64_S2_SPREAD, CFG_DMA_256x256_8W_S4_SPREAD,                           // copies spread over MFMAs
    CFG_DMA_256x192_8W_K64_S2_SPREAD, CFG_DMA_192x256_8W_K64_S2_SPREAD,                       // fewer-tile shapes
    CFG_DMA_64x32_4W_K64_S8, CFG_DMA_64x16_2W_K64_S6, CFG_DMA_64x64_4W_K64_S6,                // skinny: deep K pipelines
    CFG_DMA_256x384_8W_K64_S2_SPREAD,                                                         // all of LDS
    CFG_RING_64x32, CFG_RING_64x64, CFG_RING_32x32, CFG_RING_32x64,                          // register rings
    CFG_RING_96x64, CFG_RING_96x96, CFG_RING_128x128,                                        // register rings, mid M
    CFG_DMA_224x384_8W_K64_S2_SPREAD,                                                         // 76 copies per stage
    CFG_RING_64x128,                                                                          // register ring, wide
    CFG_COUNT
};

template <int BM, int BN, int WMW, int WNW, int EPI>
int launch_bf16_cfg(const GemmArgs& a, hipStream_t s) {
    const int out_cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const long long tiles = (long long)((a.M + BM - 1) / BM) * ((a.N + out_cols - 1) / out_cols);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WMW, WNW, EPI>), dim3((unsigned)tiles), dim3(64 * WMW * WNW), 0, s, a);
    return check_launch("gemm_bf16");
}

template <int BM, int BN, int WMW, int WNW, int BK, int STAGES, int MINW, int FEED, int EPI>
int launch_dma(const GemmArgs& a, hipStream_t s) {
    if constexpr (EPI == EPI_SWIGLU && (BN / WNW / 2) % 16 != 0) {
        // a wave's columns must split into whole 16-wide gate and up fragments
        return launch_dma<256, 256, 2, 4, 64, 2, 2, 1, EPI>(a, s);
    } else {
        const int out_cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
        const long long tiles = (long long)((a.M + BM - 1) / BM) * ((a.N + out_cols - 1) / out_cols);
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, WMW, WNW, BK, STAGES, MINW, FEED, EPI>), dim3((unsigned)tiles),
                           dim3(64 * WMW * WNW), 0, s, a);
        return check_launch("gemm_bf16_dma");
    }
}

// Register rings: BIG tiles (96 rows or more) take 128-deep K steps, two in flight, twice the computing waves
// loading; the small ones 256-deep steps, two in flight, four times the computing waves loading (128-deep,
// four in flight, twice the waves, when K is not a multiple of 256).  A K that is not a multiple of 128 takes
// 64-deep steps, 8 in flight, every wave computing.  The MFMA sequence is the same on every path.
template <int BM, int BN, int WMW, int WNW, bool BIG, int EPI>
int launch_ring(const GemmArgs& a, hipStream_t s) {
    if constexpr (EPI == EPI_SWIGLU && (BN / WNW / 2) % 16 != 0) {
        return launch_ring<BM, 2 * BN, WMW, WNW, BIG, EPI>(a, s);      // gate/up need 16-wide halves per wave
    } else {
        const int out_cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
        const dim3 grid((unsigned)((long long)((a.M + BM - 1) / BM) * ((a.N + out_cols - 1) / out_cols)));
        constexpr int W = 64 * WMW * WNW;
        if constexpr (!BIG) {
            if (a.K % 256 == 0) {
                hipLaunchKernelGGL((gemm_bf16_ring_kernel<BM, BN, WMW, WNW, 2, EPI, 256, 4>), grid, dim3(4 * W), 0, s, a);
                return check_launch("gemm_bf16_ring");
            }
        }
        if (a.K % 128 == 0)
            hipLaunchKernelGGL((gemm_bf16_ring_kernel<BM, BN, WMW, WNW, BIG ? 2 : 4, EPI, 128, 2>), grid, dim3(2 * W), 0, s, a);
        else
            hipLaunchKernelGGL((gemm_bf16_ring_kernel<BM, BN, WMW, WNW, 8, EPI, 64, 1>), grid, dim3(W), 0, s, a);
        return check_launch("gemm_bf16_ring");
    }
}

// GEMMs too small for a full round of big tiles (decode-heavy iterations: M of a few
// hundred rows or less).  Each workgroup walks all of K (one MFMA chain per output,
// K is never split), so the busiest CU's operand bytes over the rate one CU takes
// them in bound the time: estimated t = max(weight bytes at 6 TB/s, busiest x K
// tiles x tile bytes / min(cu_rate, wg_rate x busiest)), busiest = ceil(tiles /
// CUs) workgroups on the fullest CU.  wg_rate (one workgroup alone on a CU) and
// cu_rate (the CU's ceiling with several) are measured on MI355X, in GB/s: 128 x
// 128 register-staged 42 / 55; 64 x 32 and 64 x 64 DMA-fed with 8 and 6 stages 40
// and 44, 256 x 256 DMA-fed 40 (one per CU: their rings fill LDS); the
// register-ring tiles (128- or 256-deep steps) 50 / 60 at 32 x 32 and 53 / 70
// for the larger ones (with loading-only waves beside the computing ones), 53 /
// 65 for 96 x 64 and 128 x 128 (fitted to the measured best tile of the 8B shapes
// at 8 to 2000 rows: QKV at 385-480 rows, attention-out and FFN2 at 513-768 and
// SwiGLU at 65-96 then take 128 x 128 rings, 3-16% faster).  The 96- and
// 128-row rings serve the few-hundred-row GEMMs of an iteration in which a prompt
// joins the decodes (8B shapes at 330 rows: QKV 48 -> 32 us on 96 x 96 tiles,
// FFN2 114 -> 82 us on 96 x 64).  Up to 256 rows the big tile competes here too (an
// LM head over 64 rows streams its 1 GB of weights faster from 64 x 64 rings).  A
// 64-deep K tile of a BM x BN workgroup is (BM + BN) x 128 bytes.  SwiGLU needs
// 16-wide gate and up halves per wave, which the 32-column tiles do not have.
// E.g. the 8B-shaped FFN2 (N 4096, K 14336) at M 64 takes the 32 x 32 ring: 256
// tiles, one per CU, 1.84 MB each: ~37 us instead of 53 us with 64 x 32 tiles.
// The 64 x 128 ring (128-deep steps) comes before the 96- and 128-row rings, so it
// takes the estimates it ties with them (measured 5-10% faster there: QKV at 193
// to 320 rows, attention-out and FFN2 at 385 to 512), and it wins where both it
// and 64 x 64 sit at the weight bound but it moves fewer bytes per CU: the LM head
// over 64 rows (196 -> 182 us) and the SwiGLU FFN1 at 33 to 64 rows (one 1.5 MB
// tile per CU for 224 of them, against two 1 MB tiles on 192: 50.3 -> 49.3 us).
int pick_small(const GemmArgs& a, int epi) {
    struct Cand { int cfg, bm, bn; double wg_gbs, cu_gbs; };
    constexpr int NC = 12;
    const Cand cands[NC] = {{CFG_128x128_4W, 128, 128, 42.0, 55.0},
                            {CFG_DMA_256x256_8W_K64_S2, 256, 256, 40.0, 40.0},
                            {CFG_DMA_64x32_4W_K64_S8, 64, 32, 40.0, 40.0},
                            {CFG_DMA_64x64_4W_K64_S6, 64, 64, 44.0, 44.0},
                            {CFG_RING_64x32, 64, 32, 53.0, 70.0},
                            {CFG_RING_64x64, 64, 64, 53.0, 70.0},
                            {CFG_RING_32x32, 32, 32, 50.0, 60.0},
                            {CFG_RING_32x64, 32, 64, 53.0, 70.0},
                            {CFG_RING_64x128, 64, 128, 53.0, 70.0},
                            {CFG_RING_96x64, 96, 64, 53.0, 65.0},
                            {CFG_RING_96x96, 96, 96, 53.0, 70.0},
                            {CFG_RING_128x128, 128, 128, 53.0, 65.0}};
    const int cus = num_cus();
    const double nk = (double)a.K / 64.0;
    const double wbytes = (double)(epi == EPI_SWIGLU ? 2 * a.N : a.N) * a.K * 2.0;
    int best = CFG_128x128_4W;
    double best_t = 0.0, best_cu = 0.0;
    for (int c = 0; c < NC; ++c) {
        const Cand& k = cands[c];
        if (epi == EPI_SWIGLU && k.bn == 32) continue;
        const int out_cols = (epi == EPI_SWIGLU) ? k.bn / 2 : k.bn;
        const long long tiles = (long long)((a.M + k.bm - 1) / k.bm) * ((a.N + out_cols - 1) / out_cols);
        const double busiest = (double)((tiles + cus - 1) / cus);
        const double bytes = busiest * nk * (k.bm + k.bn) * 128.0;
        const double rate = std::min(k.cu_gbs, k.wg_gbs * busiest) * 1e3;        // bytes per us
        const double t_cu = bytes / rate;
        const double t = std::max(t_cu, wbytes / 6e6);
        // ties (both at the weight bound) go to the lighter per-CU load
        if (c == 0 || t < best_t || (t == best_t && t_cu < best_cu)) { best = k.cfg; best_t = t; best_cu = t_cu; }
    }
    return best;
}

// Pick the tile.  Small GEMMs: pick_small.  Otherwise DMA-fed tiles of 64-deep
// K: among 256x256, 256x192, 192x256, 256x384 and 224x384 the one with the
// least estimated time, rounds x tile area x feed factor, where rounds =
// ceil(tiles / CUs) (one such workgroup per CU: a partial last round costs a
// whole one) and the feed factor is the measured time per unit of tile area
// relative to 256x256 on MI355X (1.083 for the 192-wide tiles, which move more
// bytes per flop; 0.956 for 256x384, which moves fewer; 1.02 for 224x384,
// whose 76 copies per stage split unevenly over the 8 waves).  E.g. 3741 x
// 6144 (QKV) takes 256x384 (240 tiles, one round) over 256x192 (480 tiles, two
// rounds); the FFN1 gate/up GEMM (28672 W rows) takes 224x384: 1275 tiles fill
// exactly 5 rounds, against 7 rounds of 1680 256x256 tiles (the last 56% full;
// measured 675 against 706 us).  Copies are spread over the MFMAs.  Every
// configuration sums each output's K in the same order with the same MFMA, so
// the choice never changes a result bit.
int pick_cfg(const GemmArgs& a, int epi) {
    const char* e = getenv("SB_GEMM_CFG");             // tuning / test override: a CFG_* index
    if (e && *e) {
        const int forced = atoi(e);
        if (forced >= 0 && forced < CFG_COUNT) return forced;
    }
    const int ncols = (epi == EPI_SWIGLU) ? 2 * a.N : a.N;
    const long long big = (long long)((a.M + 255) / 256) * ((ncols + 255) / 256);
    if (big < 128 || a.M <= 256) return pick_small(a, epi);
    struct Cand { int cfg, bm, bn; double feed; };
    constexpr int NC = 5;
    const Cand cands[NC] = {{CFG_DMA_256x256_8W_K64_S2_SPREAD, 256, 256, 1.0},
                            {CFG_DMA_256x192_8W_K64_S2_SPREAD, 256, 192, 1.083},
                            {CFG_DMA_192x256_8W_K64_S2_SPREAD, 192, 256, 1.083},
                            {CFG_DMA_256x384_8W_K64_S2_SPREAD, 256, 384, 0.956},
                            {CFG_DMA_224x384_8W_K64_S2_SPREAD, 224, 384, 1.02}};
    const int cus = num_cus();
    int best = cands[0].cfg;
    double best_cost = 0.0;
    for (int c = 0; c < NC; ++c) {
        const Cand& k = cands[c];
        if (epi == EPI_SWIGLU && k.bn == 192) continue;           // gate/up need 16-wide halves per wave
        if (epi == EPI_GELU && k.bn == 384) continue;             // erf's registers do not fit beside 168+ accumulators
        const long long tiles = (long long)((a.M + k.bm - 1) / k.bm) * ((ncols + k.bn - 1) / k.bn);
        const long long rounds = (tiles + cus - 1) / cus;
        const double cost = (double)rounds * k.bm * k.bn * k.feed;
        if (c == 0 || cost < best_cost) { best = k.cfg; best_cost = cost; }
    }
    return best;
}

template <int EPI>
int launch_bf16(const GemmArgs& a, hipStream_t s) {
    switch (pick_cfg(a, EPI)) {
        case CFG_256x256_4W: return launch_bf16_cfg<256, 256, 2, 2, EPI>(a, s);
        case CFG_256x256_8W: return launch_bf16_cfg<256, 256, 2, 4, EPI>(a, s);
        case CFG_256x128_4W: return launch_bf16_cfg<256, 128, 2, 2, EPI>(a, s);
        case CFG_128x256_4W: return launch_bf16_cfg<128, 256, 2, 2, EPI>(a, s);
        case CFG_DMA_256x256_8W_S4: return launch_dma<256, 256, 2, 4, 32, 4, 2, 0, EPI>(a, s);
        case CFG_DMA_256x128_4W_S3: return launch_dma<256, 128, 2, 2, 32, 3, 2, 0, EPI>(a, s);
        case CFG_DMA_128x256_4W_S3: return launch_dma<128, 256, 2, 2, 32, 3, 2, 0, EPI>(a, s);
        case CFG_DMA_256x256_8W_S5: return launch_dma<256, 256, 2, 4, 32, 5, 2, 0, EPI>(a, s);
        case CFG_DMA_256x256_8W_K64_S2: return launch_dma<256, 256, 2, 4, 64, 2, 2, 0, EPI>(a, s);
        case CFG_DMA_256x256_4W_K64_S2: return launch_dma<256, 256, 2, 2, 64, 2, 1, 0, EPI>(a, s);
        case CFG_DMA_256x256_8W_K64_S2_SPREAD: return launch_dma<256, 256, 2, 4, 64, 2, 2, 1, EPI>(a, s);
        case CFG_DMA_256x256_8W_S4_SPREAD: return launch_dma<256, 256, 2, 4, 32, 4, 2, 1, EPI>(a, s);
        case CFG_DMA_256x192_8W_K64_S2_SPREAD: return launch_dma<256, 192, 2, 4, 64, 2, 2, 1, EPI>(a, s);
        case CFG_DMA_192x256_8W_K64_S2_SPREAD: return launch_dma<192, 256, 2, 4, 64, 2, 2, 1, EPI>(a, s);
        case CFG_DMA_64x32_4W_K64_S8: return launch_dma<64, 32, 2, 2, 64, 8, 2, 0, EPI>(a, s);
        case CFG_DMA_64x16_2W_K64_S6: return launch_dma<64, 16, 2, 1, 64, 6, 2, 0, EPI>(a, s);
        case CFG_DMA_64x64_4W_K64_S6: return launch_dma<64, 64, 2, 2, 64, 6, 2, 0, EPI>(a, s);
        case CFG_DMA_256x384_8W_K64_S2_SPREAD: return launch_dma<256, 384, 2, 4, 64, 2, 2, 1, EPI>(a, s);
        case CFG_RING_64x32: return launch_ring<64, 32, 2, 2, false, EPI>(a, s);
        case CFG_RING_64x64: return launch_ring<64, 64, 2, 2, false, EPI>(a, s);
        case CFG_RING_32x32: return launch_ring<32, 32, 2, 2, false, EPI>(a, s);
        case CFG_RING_32x64: return launch_ring<32, 64, 2, 2, false, EPI>(a, s);
        case CFG_RING_96x64: return launch_ring<96, 64, 2, 2, true, EPI>(a, s);
        case CFG_RING_96x96: return launch_ring<96, 96, 2, 2, true, EPI>(a, s);
        case CFG_RING_128x128: return launch_ring<128, 128, 2, 2, true, EPI>(a, s);
        case CFG_DMA_224x384_8W_K64_S2_SPREAD: return launch_dma<224, 384, 2, 4, 64, 2, 2, 1, EPI>(a, s);
        case CFG_RING_64x128: return launch_ring<64, 128, 2, 2, true, EPI>(a, s);
        default: return launch_bf16_cfg<128, 128, 2, 2, EPI>(a, s);
    }
}

template <int EPI>
int launch_f32(const GemmArgs& a, hipStream_t s) {
    const int out_cols = (EPI == EPI_SWIGLU) ? 32 : 64;
    const long long tiles = (long long)((a.M + 63) / 64) * ((a.N + out_cols - 1) / out_cols);
    hipLaunchKernelGGL((gemm_f32_mfma_kernel<EPI>), dim3((unsigned)tiles), dim3(256), 0, s, a);
    return check_launch("gemm_f32");
}

}  // namespace

int num_cus() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

int launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s) {
    if (a.M <= 0) return SB_OK;
    if (a.N <= 0 || a.K <= 0 || !a.A || !a.W || !a.C) return fail(SB_ERR_INVALID, "gemm: bad arguments");
    // the kernels index every operand with 32-bit element offsets
    const long long w_rows = epi == EPI_SWIGLU ? 2LL * a.F : (long long)a.N;
    const long long lim = 1LL << 31;
    if ((long long)a.M * a.lda >= lim || w_rows * a.ldw >= lim || (long long)a.M * a.ldc >= lim)
        return fail(SB_ERR_INVALID, "gemm: an operand spans 2^31 elements or more (M %d, lda %lld, W rows %lld, ldw %lld, ldc %lld)",
                    a.M, (long long)a.lda, w_rows, (long long)a.ldw, (long long)a.ldc);
    if (dtype == SB_BF16) {
        if (a.K % 64 || a.lda % 8 || a.ldw % 8) return fail(SB_ERR_INVALID, "bf16 gemm needs K %% 64 == 0 and 16-byte aligned rows");
        switch (epi) {
            case EPI_STORE: return launch_bf16<EPI_STORE>(a, s);
            case EPI_GELU: return launch_bf16<EPI_GELU>(a, s);
            case EPI_RESID: return launch_bf16<EPI_RESID>(a, s);
            case EPI_SWIGLU: return launch_bf16<EPI_SWIGLU>(a, s);
        }
    } else {
        if (a.K % 16 || a.lda % 4 || a.ldw % 4) return fail(SB_ERR_INVALID, "fp32 gemm needs K %% 16 == 0 and 16-byte aligned rows");
        switch (epi) {
            case EPI_STORE: return launch_f32<EPI_STORE>(a, s);
            case EPI_GELU: return launch_f32<EPI_GELU>(a, s);
            case EPI_RESID: return launch_f32<EPI_RESID>(a, s);
            case EPI_SWIGLU: return launch_f32<EPI_SWIGLU>(a, s);
        }
    }
    return fail(SB_ERR_INVALID, "gemm: unknown epilogue %d", epi);
}

}  // namespace sb
