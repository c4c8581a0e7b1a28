// Token-wise linear layers over the flattened [T, K] activation: C = A W^T.
//
// Selective batching runs every non-attention operator on the [sum L_i, H]
// tensor so that each weight is read once per iteration for all requests
// ("连续批处理完全拆解", section 观察; "CS349D Lecture 2", section 4.2).  T is
// arbitrary (ragged), so rows beyond T are masked; N and K come from the model.
//
// bf16: v_mfma_f32_16x16x32_bf16 tiles, 256-thread workgroups (2 x 2 waves),
// double-buffered LDS stages fed by 16-byte global loads, padded LDS rows
// (no bank conflicts on the 16-byte operand reads), XCD-aware tile order.
// fp32: a plain LDS-tiled FMA kernel with a fixed, sequential K order.
// Epilogues fuse bias, exact GeLU, SwiGLU (SiLU(gate) * up) or the residual
// add into the fp32 stream x.
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

// ================================================================== bf16 MFMA
// Workgroup tile BM x BN (BN counts W rows; for SwiGLU half are gate rows,
// half up rows), 4 waves as 2 x 2, wave tile WM x WN of 16 x 16 MFMA blocks.
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
    constexpr int BK = 64, LDSK = BK + 8;            // 144-byte rows: conflict-free 16-byte reads
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MI = WM / 16, NI = WN / 16;
    constexpr int CH = BK / 8;                       // 16-byte chunks per row
    constexpr int A_CH = BM * CH / 256, B_CH = BN * CH / 256;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDSK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDSK];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int out_cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int tiles_n = (a.N + out_cols - 1) / out_cols;
    const int total = tiles_m * tiles_n;
    const int pid = xcd_remap(blockIdx.x, total);
    // grouped order: GROUP_M row tiles sweep the column tiles together (L2 reuse of both operands)
    constexpr int GROUP_M = 8;
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
        const int c = tid + 256 * q, row = c / CH, kc = (c % CH) * 8;
        pa[q] = A + (long long)min(m0 + row, a.M - 1) * a.lda + kc;
    }
#pragma unroll
    for (int q = 0; q < B_CH; ++q) {
        const int c = tid + 256 * q, row = c / CH, kc = (c % CH) * 8;
        int gr;
        if (EPI == EPI_SWIGLU) {
            // LDS rows [wn*WN, wn*WN + WN/2) are gate rows, the next WN/2 the matching up rows
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
            const int c = tid + 256 * q;
            *(u32x4*)&As[buf][(c / CH) * LDSK + (c % CH) * 8] = ra[q];
        }
#pragma unroll
        for (int q = 0; q < B_CH; ++q) {
            const int c = tid + 256 * q;
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
            bf16x8 af[MI], bfr[NI];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                af[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)&As[buf][(wm * WM + i * 16 + lrow) * LDSK + ks * 32 + lk]);
#pragma unroll
            for (int j = 0; j < NI; ++j)
                bfr[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)&Bs[buf][(wn * WN + j * 16 + lrow) * LDSK + ks * 32 + lk]);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) stash(buf ^ 1);
        __syncthreads();
    }

    // 16x16 MFMA result: lane holds rows 4*(lane/16) + r, column lane % 16
    const int rbase = m0 + wm * WM + (lane >> 4) * 4;
    if (EPI == EPI_SWIGLU) {
        const int fbase = tn * (BN / 2) + wn * (WN / 2) + lrow;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI / 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = rbase + i * 16 + r, f = fbase + j * 16;
                    if (m < a.M && f < a.N) swiglu_store<SB_BF16>(a, m, f, acc[i][j][r], acc[i][j + NI / 2][r]);
                }
    } else {
        const int nbase = tn * BN + wn * WN + lrow;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = rbase + i * 16 + r, n = nbase + j * 16;
                    if (m < a.M && n < a.N) epi_store<SB_BF16, EPI>(a, m, n, acc[i][j][r]);
                }
    }
}

// ================================================================== fp32 FMA
// 64 x 64 tile (for SwiGLU: 32 gate + 32 up columns), 4 x 4 outputs per
// thread, K in steps of 16 through LDS.  Each output's K sum runs in
// ascending k, independent of M and of the tile a row falls in.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
    __shared__ float As[16][64 + 4];
    __shared__ float Bs[16][64 + 4];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int out_cols = (EPI == EPI_SWIGLU) ? 32 : 64;
    const int tiles_n = (a.N + out_cols - 1) / out_cols;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * 64;
    const float* A = (const float*)a.A;
    const float* W = (const float*)a.W;
    const int lr = tid >> 2, lk = (tid & 3) * 4;
    const float* pa = A + (long long)min(m0 + lr, a.M - 1) * a.lda + lk;
    int br;
    if (EPI == EPI_SWIGLU) {
        const int j = lr & 3, f = tn * 32 + (lr >> 2) * 2 + (j & 1);
        br = min(f, a.N - 1) + (j >= 2 ? a.F : 0);
    } else {
        br = min(tn * 64 + lr, a.N - 1);
    }
    const float* pb = W + (long long)br * a.ldw + lk;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < a.K; k0 += 16) {
        const float4 va = *(const float4*)(pa + k0);
        const float4 vb = *(const float4*)(pb + k0);
        As[lk + 0][lr] = va.x; As[lk + 1][lr] = va.y; As[lk + 2][lr] = va.z; As[lk + 3][lr] = va.w;
        Bs[lk + 0][lr] = vb.x; Bs[lk + 1][lr] = vb.y; Bs[lk + 2][lr] = vb.z; Bs[lk + 3][lr] = vb.w;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= a.M) continue;
        if (EPI == EPI_SWIGLU) {
            // columns tx*4 + {0,1} are gate, tx*4 + {2,3} the matching up values
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int f = tn * 32 + tx * 2 + j;
                if (f < a.N) swiglu_store<SB_F32>(a, m, f, acc[i][j], acc[i][j + 2]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = tn * 64 + tx * 4 + j;
                if (n < a.N) epi_store<SB_F32, EPI>(a, m, n, acc[i][j]);
            }
        }
    }
}

template <int EPI>
int launch_bf16(const GemmArgs& a, hipStream_t s) {
    constexpr int BM = 128, BN = 128;
    const int out_cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const long long tiles = (long long)((a.M + BM - 1) / BM) * ((a.N + out_cols - 1) / out_cols);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, EPI>), dim3((unsigned)tiles), dim3(256), 0, s, a);
    return check_launch("gemm_bf16");
}

template <int EPI>
int launch_f32(const GemmArgs& a, hipStream_t s) {
    const int out_cols = (EPI == EPI_SWIGLU) ? 32 : 64;
    const long long tiles = (long long)((a.M + 63) / 64) * ((a.N + out_cols - 1) / out_cols);
    hipLaunchKernelGGL((gemm_f32_kernel<EPI>), dim3((unsigned)tiles), dim3(256), 0, s, a);
    return check_launch("gemm_f32");
}

}  // namespace

int launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s) {
    if (a.M <= 0) return SB_OK;
    if (a.N <= 0 || a.K <= 0 || !a.A || !a.W || !a.C) return fail(SB_ERR_INVALID, "gemm: bad arguments");
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
