// Token-wise elementwise kernels and the device entry points of libsb:
// embedding, LayerNorm / RMSNorm, RoPE + K/V append, greedy argmax, and the
// sb_embed / sb_layer_step / sb_lm_argmax orchestration of one selective-
// batched iteration ("连续批处理完全拆解", Figure 5 data flow; "CS349D Lecture
// 2", section 4.2).  All of them are HBM-bound: one row per workgroup,
// 16-byte accesses along the row where the layout allows.
#include <cmath>
#include <mutex>

#include "sb_device.h"
#include "sb_ops.h"

namespace sb {

int launch_attention(const sb_model_dims* dims, const sb_ragged* rg, const void* kplane, const void* vplane,
                     long long arena, const void* qkv, void* out, float* part_o, float* part_ml, hipStream_t s);

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SB_ERR_DEVICE, "%s launch: %s", what, hipGetErrorString(e));
    return SB_OK;
}

// ------------------------------------------------------------------ timing
namespace {
struct TimingState {
    std::mutex mu;
    uint32_t mask = 0;                     // bit k: time launches of class k
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[SB_K_COUNT];
    std::vector<hipEvent_t> open[SB_K_COUNT];
};
TimingState& timing() {
    static TimingState t;
    return t;
}
}  // namespace

void timing_begin(int kind, hipStream_t s) {
    auto& T = timing();
    if (!(T.mask >> kind & 1u)) return;
    std::lock_guard<std::mutex> g(T.mu);
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return;
    hipEventRecord(e, s);
    T.open[kind].push_back(e);
}

void timing_end(int kind, hipStream_t s) {
    auto& T = timing();
    if (!(T.mask >> kind & 1u)) return;
    std::lock_guard<std::mutex> g(T.mu);
    if (T.open[kind].empty()) return;
    hipEvent_t b = T.open[kind].back();
    T.open[kind].pop_back();
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return;
    hipEventRecord(e, s);
    T.ev[kind].push_back({b, e});
}

// ------------------------------------------------------------------ kernels
namespace {

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
    return t;
}

// Four consecutive elements of a dtype row as one 8-byte access (bf16) or one 16-byte access
// (fp32); the pointer is aligned to the access.
template <int DT>
__device__ __forceinline__ void load4(const typename Store<DT>::T* p, float (&v)[4]) {
    if constexpr (DT == SB_BF16) {
        const u32x2 w = *(const u32x2*)p;
        v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
        v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
        const float4 w = *(const float4*)p;
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
    }
}
template <int DT>
__device__ __forceinline__ void store4(typename Store<DT>::T* p, const float (&v)[4]) {
    if constexpr (DT == SB_BF16) {
        *(u32x2*)p = u32x2{(uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16),
                           (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16)};
    } else {
        *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// x[t] = E[id_t] (+ P[pos_t]) in fp32.  A negative id -(1 + j) refers to the
// token the previous iteration generated in its batch row j (prev[j], still on
// the device); ids are clamped into the tables so no value can read outside them.
template <int DT>
__global__ __launch_bounds__(256) void embed_kernel(const int* ids, const int* pos, const void* tok, const void* pe,
                                                    const int* prev, int prev_n, int vocab, float* x, int H, int vec) {
    using T = typename Store<DT>::T;
    const int t = blockIdx.x;
    int id = ids[t];
    if (id < 0) {
        const int j = -1 - id;
        id = (prev && j < prev_n) ? prev[j] : 0;
    }
    id = min(max(id, 0), vocab - 1);
    const T* e = (const T*)tok + (long long)id * H;
    const T* p = pe ? (const T*)pe + (long long)pos[t] * H : nullptr;
    float* xo = x + (long long)t * H;
    if (vec) {
        // four elements per access (8-byte bf16 / 16-byte fp32 loads, 16-byte stores), every load of the row
        // issued before the first store
        constexpr int NV = 4;                         // hidden <= 4096: at most 4 pieces per thread
        const int n4 = H / 4;
        float v[NV][4];
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int i = threadIdx.x + q * blockDim.x;
            if (i < n4) {
                load4<DT>(e + 4 * i, v[q]);
                if (p) {
                    float w[4];
                    load4<DT>(p + 4 * i, w);
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[q][c] += w[c];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int i = threadIdx.x + q * blockDim.x;
            if (i < n4) *(float4*)(xo + 4 * i) = make_float4(v[q][0], v[q][1], v[q][2], v[q][3]);
        }
        return;
    }
    for (int i = threadIdx.x; i < H; i += blockDim.x) {
        float v = Store<DT>::ld(e + i);
        if (p) v += Store<DT>::ld(p + i);
        xo[i] = v;
    }
}


// LayerNorm (kind 0) or RMSNorm (kind 1) of fp32 rows into dtype rows; fp32
// statistics, two passes over registers (mean, then centred second moment).
// Every kernel below sums a row in one canonical order, so a row's result does
// not depend on how many rows were normalised together (which kernel ran):
// piece i of the row (elements 4i .. 4i+3) contributes (a + b) + (c + d) (its
// square terms likewise); lane l of 64 adds the pieces l, l + 64, l + 128, ...
// in ascending order; the 64 lane sums meet in an xor butterfly.
//   norm_kernel<.., WPR = 1>: one wave per row (four rows per workgroup), the
//     order above directly (hidden <= 256 PER).
//   norm_kernel<.., WPR = 4>: one row per workgroup (hidden > 1024): a quarter
//     of the dependent loads per lane and several small workgroups per CU, so
//     many rows' loads are in flight at once; the 256 threads leave their piece
//     sums in LDS and one wave adds them in the order above.
// 16-byte loads along the row.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Raw 4-element piece of a dtype row (8 bytes of bf16 or 16 of fp32), widened later.
template <int DT>
struct Raw4 { using T = u32x2; };
template <>
struct Raw4<SB_F32> { using T = float4; };
template <int DT>
__device__ __forceinline__ void widen4(const typename Raw4<DT>::T& w, float (&v)[4]) {
    if constexpr (DT == SB_BF16) {
        v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
        v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
    }
}

// The per-piece terms and the output of one piece, shared by every norm kernel.
__device__ __forceinline__ float piece_sum(const float4& v) { return (v.x + v.y) + (v.z + v.w); }
__device__ __forceinline__ float piece_sq(const float4& v, float mean) {
    const float a = v.x - mean, b = v.y - mean, c = v.z - mean, d = v.w - mean;
    return (a * a + b * b) + (c * c + d * d);
}
template <int DT>
__device__ __forceinline__ void norm_piece_out(typename Store<DT>::T* o, const float4& v, float mean, float rstd,
                                               const typename Raw4<DT>::T& gr, const typename Raw4<DT>::T* br) {
    const float xs[4] = {v.x, v.y, v.z, v.w};
    float gv[4], bv[4] = {0.f, 0.f, 0.f, 0.f}, y[4];
    widen4<DT>(gr, gv);
    if (br) widen4<DT>(*br, bv);
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = (xs[c] - mean) * rstd * gv[c] + bv[c];
    store4<DT>(o, y);
}

constexpr int kNormMaxPieces = 12288 / 4;

template <int DT, int PER, int WPR>
__global__ __launch_bounds__(256) void norm_kernel(const float* x, const int* row_map, const void* gam, const void* bet,
                                                   void* out, int rows, int H, int kind, float eps) {
    using T = typename Store<DT>::T;
    using R = typename Raw4<DT>::T;
    __shared__ float red[WPR == 1 ? 1 : kNormMaxPieces + 1];
    constexpr int LANES = 64 * WPR;                        // threads per row
    const int lane = threadIdx.x % LANES;
    const int r = blockIdx.x * (4 / WPR) + threadIdx.x / LANES;
    if (r >= rows) return;                                 // whole rows only: block-uniform when WPR = 4
    const long long src = row_map ? row_map[r] : r;
    const float4* xr = (const float4*)(x + src * H);
    const T* g = (const T*)gam;
    const T* b = (const T*)bet;
    const int n4 = H / 4;
    // the row, the gain and the shift are all requested before the first reduction
    float4 v[PER];
    R gr[PER], br[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int i = lane + LANES * q;
        if (i < n4) {
            v[q] = xr[i];
            gr[q] = *(const R*)(g + 4 * i);
            if (b) br[q] = *(const R*)(b + 4 * i);
        }
    }
    // the canonical row sum of term(q) over this thread's pieces
    auto row_sum = [&](auto term) {
        if constexpr (WPR == 1) {
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < PER; ++q)
                if (lane + LANES * q < n4) s += term(q);
            return wave_sum(s);
        } else {
#pragma unroll
            for (int q = 0; q < PER; ++q)
                if (lane + LANES * q < n4) red[lane + LANES * q] = term(q);
            __syncthreads();
            if (threadIdx.x < 64) {
                float s = 0.f;
                for (int i = threadIdx.x; i < n4; i += 64) s += red[i];
                s = wave_sum(s);
                if (threadIdx.x == 0) red[kNormMaxPieces] = s;
            }
            __syncthreads();
            const float tot = red[kNormMaxPieces];
            __syncthreads();                               // red is rewritten by the next sum
            return tot;
        }
    };
    const float mean = kind == 0 ? row_sum([&](int q) { return piece_sum(v[q]); }) / H : 0.f;
    const float rstd = 1.0f / sqrtf(row_sum([&](int q) { return piece_sq(v[q], mean); }) / H + eps);
    T* o = (T*)out + (long long)r * H;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int i = lane + LANES * q;
        if (i < n4) norm_piece_out<DT>(o + 4 * i, v[q], mean, rstd, gr[q], b ? &br[q] : nullptr);
    }
}

// Per token: rotate q (in place in qkv) and k by the token's position
// (Llama-style, rotate-half pairs (i, i + d/2), angle pos * theta^(-2i/d),
// evaluated in double precision once per token), then append k and v to the
// K/V manager's arenas at the token's slot (k rotated there; qkv's k part is
// left as it was).  A rotation item is 8 consecutive dims of one half-head with
// the matching 8 of the other half (q heads with rotation, k heads always):
// 16-byte accesses in bf16.  Every thread issues the loads of its first items
// before the token's cos/sin are evaluated, so the double-precision evaluation
// overlaps the memory latency.  V is appended per 8-slot block (below).
constexpr int kRopeMaxHalf = 64;        // head_dim <= 128
constexpr int kRopeItemsPerThread = 2;  // items a thread has in flight at once

template <int DT>
struct Piece8 {                          // 8 consecutive elements, raw
    u32x4 r[DT == SB_BF16 ? 1 : 2];
};
template <int DT>
__device__ __forceinline__ Piece8<DT> ld_piece(const typename Store<DT>::T* p) {
    Piece8<DT> x;
    x.r[0] = *(const u32x4*)p;
    if constexpr (DT != SB_BF16) x.r[1] = *(const u32x4*)(p + 4);
    return x;
}
template <int DT>
__device__ __forceinline__ void st_piece(typename Store<DT>::T* p, const Piece8<DT>& x) {
    *(u32x4*)p = x.r[0];
    if constexpr (DT != SB_BF16) *(u32x4*)(p + 4) = x.r[1];
}
template <int DT>
__device__ __forceinline__ void piece_to_f32(const Piece8<DT>& x, float (&v)[8]) {
    if constexpr (DT == SB_BF16) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            v[2 * c] = __uint_as_float(x.r[0][c] << 16);
            v[2 * c + 1] = __uint_as_float(x.r[0][c] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) { v[c] = __uint_as_float(x.r[0][c]); v[4 + c] = __uint_as_float(x.r[1][c]); }
    }
}
template <int DT>
__device__ __forceinline__ Piece8<DT> f32_to_piece(const float (&v)[8]) {
    Piece8<DT> x;
    if constexpr (DT == SB_BF16) {
#pragma unroll
        for (int c = 0; c < 4; ++c) x.r[0][c] = (uint32_t)f2bf(v[2 * c]) | ((uint32_t)f2bf(v[2 * c + 1]) << 16);
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) { x.r[0][c] = __float_as_uint(v[c]); x.r[1][c] = __float_as_uint(v[4 + c]); }
    }
    return x;
}

template <int DT>
__global__ __launch_bounds__(256) void rope_append_kernel(void* qkv, long long stride, const int* pos, const int* slot,
                                                          void* kplane, void* vplane, long long arena, int nq, int nkv,
                                                          int D, int rope, double log_theta) {
    using T = typename Store<DT>::T;
    constexpr int IPT = kRopeItemsPerThread;
    __shared__ float cs[kRopeMaxHalf], sn[kRopeMaxHalf];
    const int t = blockIdx.x, n_tok = gridDim.x;
    T* row = (T*)qkv + (long long)t * stride;
    T* K = (T*)kplane;
    T* V = (T*)vplane;
    const int half = D / 2, cph = half / 8;                 // 8-dim pieces per half-head
    const int h0 = rope ? 0 : nq;                           // first rotated head (q untouched without rotation)
    const int n_rot = (nq + nkv - h0) * cph;                // rotation items
    const long long s = slot[t];
    Piece8<DT> x1[IPT], x2[IPT];
    auto fetch = [&](int base) {
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const int w = base + j * blockDim.x + threadIdx.x;
            if (w < n_rot) {
                const T* p = row + (long long)(h0 + w / cph) * D + (w % cph) * 8;
                x1[j] = ld_piece<DT>(p);
                x2[j] = ld_piece<DT>(p + half);
            }
        }
    };
    auto process = [&](int base) {
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const int w = base + j * blockDim.x + threadIdx.x;
            if (w >= n_rot) continue;
            const int h = h0 + w / cph, i0 = (w % cph) * 8;
            Piece8<DT> y1 = x1[j], y2 = x2[j];
            if (rope) {
                float a[8], b[8], c1[8], c2[8];
                piece_to_f32<DT>(x1[j], a);
                piece_to_f32<DT>(x2[j], b);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    c1[c] = a[c] * cs[i0 + c] - b[c] * sn[i0 + c];
                    c2[c] = b[c] * cs[i0 + c] + a[c] * sn[i0 + c];
                }
                y1 = f32_to_piece<DT>(c1);
                y2 = f32_to_piece<DT>(c2);
            }
            T* p = h < nq ? row + (long long)h * D + i0 : K + ((long long)(h - nq) * arena + s) * D + i0;
            st_piece<DT>(p, y1);
            st_piece<DT>(p + half, y2);
        }
    };
    fetch(0);
    if (rope) {
        for (int i = threadIdx.x; i < half; i += blockDim.x) {
            const double inv = exp(-(2.0 * i / D) * log_theta);
            double sv, cv;
            sincos((double)pos[t] * inv, &sv, &cv);
            cs[i] = (float)cv;
            sn[i] = (float)sv;
        }
        __syncthreads();
    }
    process(0);
    for (int base = IPT * blockDim.x; base < n_rot; base += IPT * blockDim.x) {
        fetch(base);
        process(base);
    }

    // v into the blocked layout [slot / 8][dim][slot % 8].  A request's new tokens sit in consecutive
    // rows at consecutive slots, and slots are unique, so the rows after t holding slots s + 1, s + 2,
    // ... are that request's next tokens.  The token opening such a run inside one 8-slot block (its
    // slot opens the block, or the row before is not the slot before) appends the run's n (<= 8)
    // tokens: a whole block as one 16-byte piece per (head, dim) -- consecutive lanes on consecutive
    // dims, so a wave writes 1 KB of whole lines -- a partial one element by element.
    const int sl = (int)(s & 7);
    const bool lead = sl == 0 || t == 0 || slot[t - 1] != s - 1;
    if (!lead) return;
    int nxt[7];
#pragma unroll
    for (int j = 1; j < 8; ++j) nxt[j - 1] = slot[min(t + j, n_tok - 1)];
    int n = 1;
#pragma unroll
    for (int j = 1; j < 8; ++j)
        if (n == j && sl + j < 8 && t + j < n_tok && nxt[j - 1] == s + j) n = j + 1;
    const T* vr = row + (long long)(nq + nkv) * D;          // v of row t; of row t + j at + j * stride
    T* vb = V + ((s >> 3) * D << 3);                         // the block, K/V head 0
    for (int u = threadIdx.x; u < nkv * D; u += blockDim.x) {
        const int g = u / D, e = u % D;
        T* dst = vb + (long long)g * arena * D + (e << 3);
        if (n == 8) {
            T v8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v8[j] = vr[u + j * stride];
            if constexpr (DT == SB_BF16) {
                u32x4 w;
#pragma unroll
                for (int c = 0; c < 4; ++c) w[c] = (uint32_t)v8[2 * c] | ((uint32_t)v8[2 * c + 1] << 16);
                *(u32x4*)dst = w;
            } else {
                *(float4*)dst = make_float4(v8[0], v8[1], v8[2], v8[3]);
                *(float4*)(dst + 4) = make_float4(v8[4], v8[5], v8[6], v8[7]);
            }
        } else {
            for (int j = 0; j < n; ++j) dst[sl + j] = vr[u + j * stride];
        }
    }
}

// Scatter / gather of whole K/V rows [n][nkv][d] at explicit slots.
template <int DT>
__global__ __launch_bounds__(256) void kv_copy_kernel(const int* slots, void* kplane, void* vplane, long long arena,
                                                      int nkv, int D, void* k, void* v, int write) {
    using T = typename Store<DT>::T;
    const int t = blockIdx.x;
    const long long s = slots[t];
    if (s < 0 || s >= arena) return;          // a slot outside the arena is skipped, never dereferenced
    T* K = (T*)kplane;
    T* V = (T*)vplane;
    T* kr = (T*)k + (long long)t * nkv * D;
    T* vr = (T*)v + (long long)t * nkv * D;
    for (int idx = threadIdx.x; idx < nkv * D; idx += blockDim.x) {
        const int g = idx / D, e = idx % D;
        T* kp = K + ((long long)g * arena + s) * D + e;
        T* vp = V + (long long)g * arena * D + (((s >> 3) * D + e) << 3) + (s & 7);
        if (write) {
            *kp = kr[idx];
            *vp = vr[idx];
        } else {
            kr[idx] = *kp;
            vr[idx] = *vp;
        }
    }
}

// Greedy token: index of the largest logit, lowest index among equal maxima.
// One 1024-thread workgroup per row, 16-byte loads (the row is long: 128256
// logits of the 8B-shaped vocabulary), each thread scanning ascending indices.
constexpr int kArgmaxThreads = 1024;
__device__ __forceinline__ void argmax_take(float v, int i, float& bv, int& bi, int sentinel) {
    if (v > bv || (bi == sentinel && v == bv)) {   // ascending scan: keep the first maximum
        bv = v;
        bi = i;
    }
}
__global__ __launch_bounds__(kArgmaxThreads) void argmax_kernel(const float* logits, int V, int* out) {
    const int r = blockIdx.x;
    const float* x = logits + (long long)r * V;
    float bv = -INFINITY;
    int bi = V;
    if ((V & 3) == 0 && ((uintptr_t)logits & 15) == 0) {
        // 16-byte pieces k = threadIdx.x, + 1024, ... in ascending order, eight loads in flight per thread
        const float4* x4 = (const float4*)x;
        const int n4 = V / 4;
        constexpr int NB = 8;
        for (int k0 = threadIdx.x; k0 < n4; k0 += NB * kArgmaxThreads) {
            float4 v[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int k = k0 + b * kArgmaxThreads;
                if (k < n4) v[b] = x4[k];
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int k = k0 + b * kArgmaxThreads;
                if (k < n4) {
                    argmax_take(v[b].x, 4 * k, bv, bi, V);
                    argmax_take(v[b].y, 4 * k + 1, bv, bi, V);
                    argmax_take(v[b].z, 4 * k + 2, bv, bi, V);
                    argmax_take(v[b].w, 4 * k + 3, bv, bi, V);
                }
            }
        }
    } else {
        for (int i = threadIdx.x; i < V; i += kArgmaxThreads) argmax_take(x[i], i, bv, bi, V);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
        }
    }
    constexpr int NW = kArgmaxThreads / 64;
    __shared__ float sv[NW];
    __shared__ int si[NW];
    if ((threadIdx.x & 63) == 0) {
        sv[threadIdx.x >> 6] = bv;
        si[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < NW; ++w)
            if (sv[w] > bv || (sv[w] == bv && si[w] < bi)) {
                bv = sv[w];
                bi = si[w];
            }
        out[r] = bi;
    }
}

}  // namespace

int launch_norm(int dtype, int kind, int rows, int H, const float* x, const int* row_map, const void* g,
                const void* b, float eps, void* out, hipStream_t s) {
    if (rows <= 0) return SB_OK;
    if (H % 4 || H > 4 * kNormMaxPieces) return fail(SB_ERR_INVALID, "norm: hidden must be a multiple of 4 and <= 12288");
    TimedScope ts(SB_K_NORM, s);
    const dim3 block(256);
    auto go = [&](auto kern, int blocks) {
        hipLaunchKernelGGL(kern, dim3(blocks), block, 0, s, x, row_map, g, b, out, rows, H, kind, eps);
    };
    // one row per workgroup above hidden 1024, at every row count: at 3741 x 4096 17 us against 20 us for
    // waves that each walk ~2 rows with the next row's loads in flight
    const int per4 = (rows + 3) / 4;
    if (dtype == SB_BF16) {
        if (H <= 1024) go(norm_kernel<SB_BF16, 4, 1>, per4);
        else if (H <= 4096) go(norm_kernel<SB_BF16, 4, 4>, rows);
        else go(norm_kernel<SB_BF16, 12, 4>, rows);
    } else {
        if (H <= 1024) go(norm_kernel<SB_F32, 4, 1>, per4);
        else if (H <= 4096) go(norm_kernel<SB_F32, 4, 4>, rows);
        else go(norm_kernel<SB_F32, 12, 4>, rows);
    }
    return check_launch("norm");
}

int launch_rope_append(const sb_model_dims* d, const sb_ragged* rg, void* qkv, void* kp, void* vp, long long arena,
                       hipStream_t s) {
    if (rg->n_tokens <= 0) return SB_OK;
    if (d->head_dim % 16 || d->head_dim / 2 > kRopeMaxHalf)
        return fail(SB_ERR_INVALID, "rope/append: head_dim must be a multiple of 16 and <= %d", 2 * kRopeMaxHalf);
    if (((uintptr_t)qkv | (uintptr_t)kp | (uintptr_t)vp) % 16)
        return fail(SB_ERR_INVALID, "rope/append: qkv and the K/V planes must be 16-byte aligned");
    TimedScope ts(SB_K_ROPE_APPEND, s);
    const long long stride = (long long)(d->n_heads + 2 * d->n_kv_heads) * d->head_dim;
    const int rope = d->arch == SB_ARCH_LLAMA;
    const double lt = log((double)d->rope_theta);
    if (d->dtype == SB_BF16)
        hipLaunchKernelGGL(rope_append_kernel<SB_BF16>, dim3(rg->n_tokens), dim3(256), 0, s, qkv, stride, rg->tok_pos,
                           rg->tok_slot, kp, vp, arena, d->n_heads, d->n_kv_heads, d->head_dim, rope, lt);
    else
        hipLaunchKernelGGL(rope_append_kernel<SB_F32>, dim3(rg->n_tokens), dim3(256), 0, s, qkv, stride, rg->tok_pos,
                           rg->tok_slot, kp, vp, arena, d->n_heads, d->n_kv_heads, d->head_dim, rope, lt);
    return check_launch("rope_append");
}

int launch_argmax(int rows, int V, const float* logits, int* out, hipStream_t s) {
    if (rows <= 0) return SB_OK;
    TimedScope ts(SB_K_ARGMAX, s);
    hipLaunchKernelGGL(argmax_kernel, dim3(rows), dim3(kArgmaxThreads), 0, s, logits, V, out);
    return check_launch("argmax");
}

// ------------------------------------------------------------------ workspace
struct LayerWs {
    char* h;
    char* qkv;
    char* o;
    char* g;
    float* part_o;
    float* part_ml;
    char* hl;
    float* logits;
    size_t total;
};

static size_t al(size_t v) { return (v + 255) & ~(size_t)255; }

static LayerWs layer_ws(const sb_model_dims* d, char* base, int64_t T, int64_t B, int64_t P) {
    const size_t es = dtype_size(d->dtype);
    LayerWs w{};
    size_t o = 0;
    auto take = [&](size_t n) { char* p = base ? base + o : nullptr; o += al(n); return p; };
    w.h = take((size_t)T * d->hidden * es);
    w.qkv = take((size_t)T * (d->n_heads + 2 * d->n_kv_heads) * d->head_dim * es);
    w.o = take((size_t)T * d->n_heads * d->head_dim * es);
    w.g = take((size_t)T * d->ffn * es);
    w.part_o = (float*)take((size_t)P * 16 * d->head_dim * 4);
    w.part_ml = (float*)take((size_t)P * 16 * 2 * 4);
    w.hl = take((size_t)B * d->hidden * es);
    w.logits = (float*)take((size_t)B * (d->vocab > 0 ? d->vocab : 1) * 4);
    w.total = o;
    return w;
}

}  // namespace sb

using namespace sb;

extern "C" size_t sb_layer_workspace_bytes(const sb_model_dims* dims, int32_t max_tokens, int32_t max_req,
                                           int32_t max_partials) {
    if (validate_dims(dims) || max_tokens < 0 || max_req < 0 || max_partials < 0) return 0;
    return layer_ws(dims, nullptr, max_tokens, max_req, max_partials).total;
}

static int check_ws(const sb_model_dims* d, const sb_ragged* rg, size_t ws_bytes) {
    size_t need = layer_ws(d, nullptr, rg->n_tokens, rg->n_req, rg->n_partials).total;
    if (need > ws_bytes) return fail(SB_ERR_WORKSPACE, "workspace needs %zu bytes, %zu given", need, ws_bytes);
    return SB_OK;
}

extern "C" int sb_embed_chained(const sb_model_dims* dims, const sb_model_weights* w, const sb_ragged* rg,
                                const int32_t* prev_ids, int32_t prev_n, float* x, void* stream) {
    int st = validate_dims(dims);
    if (st) return st;
    if (!w || !rg || !x || !w->tok_emb || !rg->tok_ids) return fail(SB_ERR_INVALID, "sb_embed: NULL argument (token ids required)");
    if (dims->vocab <= 0) return fail(SB_ERR_INVALID, "sb_embed: vocab must be positive");
    if (prev_n < 0 || (prev_n > 0 && !prev_ids)) return fail(SB_ERR_INVALID, "sb_embed: bad previous ids");
    if (rg->n_tokens <= 0) return SB_OK;
    const void* pe = dims->arch == SB_ARCH_GPT ? w->pos_emb : nullptr;
    if (dims->arch == SB_ARCH_GPT && !pe) return fail(SB_ERR_INVALID, "sb_embed: GPT needs pos_emb");
    hipStream_t s = (hipStream_t)stream;
    TimedScope ts(SB_K_EMBED, s);
    // whole 4-element pieces, 16-byte aligned output rows and tables: the vector path (hidden <= 4096)
    const int vec = dims->hidden % 4 == 0 && dims->hidden <= 4 * 4 * 256 &&
                    (((uintptr_t)x | (uintptr_t)w->tok_emb | (uintptr_t)pe) % 16) == 0;
    if (dims->dtype == SB_BF16)
        hipLaunchKernelGGL(embed_kernel<SB_BF16>, dim3(rg->n_tokens), dim3(256), 0, s, rg->tok_ids, rg->tok_pos,
                           w->tok_emb, pe, prev_ids, prev_n, dims->vocab, x, dims->hidden, vec);
    else
        hipLaunchKernelGGL(embed_kernel<SB_F32>, dim3(rg->n_tokens), dim3(256), 0, s, rg->tok_ids, rg->tok_pos,
                           w->tok_emb, pe, prev_ids, prev_n, dims->vocab, x, dims->hidden, vec);
    return check_launch("embed");
}

extern "C" int sb_embed(const sb_model_dims* dims, const sb_model_weights* w, const sb_ragged* rg, float* x,
                        void* stream) {
    return sb_embed_chained(dims, w, rg, nullptr, 0, x, stream);
}

static int layer_gemm(const sb_model_dims* d, int epi, int kind, int M, int N, int K, const void* A, const void* W,
                      const void* bias, void* C, long long ldc, int F, hipStream_t s) {
    GemmArgs a{};
    a.M = M;
    a.N = N;
    a.K = K;
    a.A = A;
    a.lda = K;
    a.W = W;
    a.ldw = K;
    a.bias = bias;
    a.C = C;
    a.ldc = ldc;
    a.out_f32 = 0;
    a.F = F;
    TimedScope ts(kind, s);
    return launch_gemm(d->dtype, epi, a, s);
}

extern "C" int sb_layer_step(const sb_model_dims* d, const sb_layer_weights* w, const sb_ragged* rg, const sb_kv* kv,
                             int32_t layer, float* x, void* workspace, size_t ws_bytes, void* stream) {
    int st = validate_dims(d);
    if (st) return st;
    if (!w || !rg || !kv || !x || !workspace) return fail(SB_ERR_INVALID, "sb_layer_step: NULL argument");
    if (kv->d != d->head_dim || kv->nkv != d->n_kv_heads || kv->dtype != d->dtype)
        return fail(SB_ERR_INVALID, "K/V manager shape does not match the model");
    const bool gpt = d->arch == SB_ARCH_GPT;
    if (!w->ln1_g || !w->w_qkv || !w->w_o || !w->ln2_g || !w->w1 || !w->w2) return fail(SB_ERR_INVALID, "missing layer weight");
    if (gpt && (!w->ln1_b || !w->ln2_b)) return fail(SB_ERR_INVALID, "GPT layer needs LayerNorm shifts");
    if ((st = check_ws(d, rg, ws_bytes))) return st;
    if (rg->n_tokens <= 0) return SB_OK;
    void *kp, *vp;
    if ((st = sb_kv_layer_ptrs(kv, layer, &kp, &vp))) return st;
    hipStream_t s = (hipStream_t)stream;
    LayerWs ws = layer_ws(d, (char*)workspace, rg->n_tokens, rg->n_req, rg->n_partials);
    const int T = rg->n_tokens, H = d->hidden, F = d->ffn;
    const int qkv_n = (d->n_heads + 2 * d->n_kv_heads) * d->head_dim;
    const int attn_n = d->n_heads * d->head_dim;
    const int nk = gpt ? 0 : 1;
    // a4: norm 1 -> a5: QKV linear (+bias)
    if ((st = launch_norm(d->dtype, nk, T, H, x, nullptr, w->ln1_g, gpt ? w->ln1_b : nullptr, d->eps, ws.h, s))) return st;
    if ((st = layer_gemm(d, EPI_STORE, SB_K_GEMM_QKV, T, qkv_n, H, ws.h, w->w_qkv, gpt ? w->b_qkv : nullptr, ws.qkv, qkv_n, 0, s))) return st;
    // a5b/a6: RoPE (Llama) + append this step's k, v to the K/V manager
    if ((st = launch_rope_append(d, rg, ws.qkv, kp, vp, kv->arena_slots, s))) return st;
    // a7: Split -> per-request attention against K/V history -> Merge (offsets)
    if ((st = launch_attention(d, rg, kp, vp, kv->arena_slots, ws.qkv, ws.o, ws.part_o, ws.part_ml, s))) return st;
    // a8: attention-out linear + bias + residual into x
    if ((st = layer_gemm(d, EPI_RESID, SB_K_GEMM_O, T, H, attn_n, ws.o, w->w_o, gpt ? w->b_o : nullptr, x, H, 0, s))) return st;
    // a9: norm 2 -> a10: FFN1 (+bias, GeLU) or SwiGLU -> a11: FFN2 + bias + residual
    if ((st = launch_norm(d->dtype, nk, T, H, x, nullptr, w->ln2_g, gpt ? w->ln2_b : nullptr, d->eps, ws.h, s))) return st;
    if ((st = layer_gemm(d, gpt ? EPI_GELU : EPI_SWIGLU, SB_K_GEMM_FFN1, T, F, H, ws.h, w->w1, gpt ? w->b1 : nullptr, ws.g, F, F, s))) return st;
    if ((st = layer_gemm(d, EPI_RESID, SB_K_GEMM_FFN2, T, H, F, ws.g, w->w2, gpt ? w->b2 : nullptr, x, H, 0, s))) return st;
    return SB_OK;
}

extern "C" int sb_lm_argmax(const sb_model_dims* d, const sb_model_weights* w, const sb_ragged* rg, const float* x,
                            float* logits, int32_t* out_ids, void* workspace, size_t ws_bytes, void* stream) {
    int st = validate_dims(d);
    if (st) return st;
    if (!w || !rg || !x || !out_ids || !workspace || !w->lnf_g || !w->w_lm) return fail(SB_ERR_INVALID, "sb_lm_argmax: NULL argument");
    if (d->vocab <= 0) return fail(SB_ERR_INVALID, "vocab must be positive");
    const bool gpt = d->arch == SB_ARCH_GPT;
    if (gpt && !w->lnf_b) return fail(SB_ERR_INVALID, "GPT final norm needs its shift");
    if ((st = check_ws(d, rg, ws_bytes))) return st;
    if (rg->n_req <= 0) return SB_OK;
    hipStream_t s = (hipStream_t)stream;
    LayerWs ws = layer_ws(d, (char*)workspace, rg->n_tokens, rg->n_req, rg->n_partials);
    float* lg = logits ? logits : ws.logits;
    if ((st = launch_norm(d->dtype, gpt ? 0 : 1, rg->n_req, d->hidden, x, rg->last_row, w->lnf_g, gpt ? w->lnf_b : nullptr,
                          d->eps, ws.hl, s)))
        return st;
    GemmArgs a{};
    a.M = rg->n_req;
    a.N = d->vocab;
    a.K = d->hidden;
    a.A = ws.hl;
    a.lda = d->hidden;
    a.W = w->w_lm;
    a.ldw = d->hidden;
    a.bias = nullptr;
    a.C = lg;
    a.ldc = d->vocab;
    a.out_f32 = 1;
    {
        TimedScope ts(SB_K_GEMM_LM, s);
        if ((st = launch_gemm(d->dtype, EPI_STORE, a, s))) return st;
    }
    return launch_argmax(rg->n_req, d->vocab, lg, out_ids, s);
}

extern "C" int sb_forward(const sb_model_dims* d, const sb_model_weights* mw, const sb_layer_weights* layers,
                          int32_t n_layers, const sb_ragged* rg, const sb_kv* kv, const int32_t* prev_ids,
                          int32_t prev_n, float* x, float* logits, int32_t* out_ids, void* workspace,
                          size_t ws_bytes, void* stream) {
    if (n_layers < 0 || (n_layers > 0 && !layers)) return fail(SB_ERR_INVALID, "sb_forward: bad layer array");
    int st = sb_embed_chained(d, mw, rg, prev_ids, prev_n, x, stream);
    for (int32_t l = 0; !st && l < n_layers; ++l) st = sb_layer_step(d, &layers[l], rg, kv, l, x, workspace, ws_bytes, stream);
    if (!st) st = sb_lm_argmax(d, mw, rg, x, logits, out_ids, workspace, ws_bytes, stream);
    return st;
}

extern "C" int sb_kv_write(const sb_kv* kv, int32_t layer, int32_t n, const int32_t* slots, const void* k, const void* v,
                           void* stream) {
    if (!kv || (n > 0 && (!slots || !k || !v))) return fail(SB_ERR_INVALID, "sb_kv_write: NULL argument");
    if (n <= 0) return SB_OK;
    void *kp, *vp;
    int st = sb_kv_layer_ptrs(kv, layer, &kp, &vp);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    if (kv->dtype == SB_BF16)
        hipLaunchKernelGGL(kv_copy_kernel<SB_BF16>, dim3(n), dim3(256), 0, s, slots, kp, vp, kv->arena_slots, kv->nkv, kv->d,
                           (void*)k, (void*)v, 1);
    else
        hipLaunchKernelGGL(kv_copy_kernel<SB_F32>, dim3(n), dim3(256), 0, s, slots, kp, vp, kv->arena_slots, kv->nkv, kv->d,
                           (void*)k, (void*)v, 1);
    return check_launch("kv_write");
}

extern "C" int sb_kv_read(const sb_kv* kv, int32_t layer, int32_t n, const int32_t* slots, void* k, void* v, void* stream) {
    if (!kv || (n > 0 && (!slots || !k || !v))) return fail(SB_ERR_INVALID, "sb_kv_read: NULL argument");
    if (n <= 0) return SB_OK;
    void *kp, *vp;
    int st = sb_kv_layer_ptrs(kv, layer, &kp, &vp);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    if (kv->dtype == SB_BF16)
        hipLaunchKernelGGL(kv_copy_kernel<SB_BF16>, dim3(n), dim3(256), 0, s, slots, kp, vp, kv->arena_slots, kv->nkv, kv->d, k, v, 0);
    else
        hipLaunchKernelGGL(kv_copy_kernel<SB_F32>, dim3(n), dim3(256), 0, s, slots, kp, vp, kv->arena_slots, kv->nkv, kv->d, k, v, 0);
    return check_launch("kv_read");
}

// ------------------------------------------------------------------ timing ABI
extern "C" int sb_timing_enable(int32_t mask) {
    timing().mask = (uint32_t)mask;
    return SB_OK;
}

extern "C" int sb_timing_read(int32_t k, double* total_ms, int64_t* count) {
    if (k < 0 || k >= SB_K_COUNT) return fail(SB_ERR_INVALID, "unknown kernel class %d", k);
    auto& T = timing();
    std::lock_guard<std::mutex> g(T.mu);
    double tot = 0;
    for (auto& p : T.ev[k]) {
        if (hipEventSynchronize(p.second) != hipSuccess) return fail(SB_ERR_DEVICE, "event sync failed");
        float ms = 0;
        if (hipEventElapsedTime(&ms, p.first, p.second) != hipSuccess) return fail(SB_ERR_DEVICE, "event time failed");
        tot += ms;
    }
    if (total_ms) *total_ms = tot;
    if (count) *count = (int64_t)T.ev[k].size();
    return SB_OK;
}

extern "C" int sb_timing_reset(void) {
    auto& T = timing();
    std::lock_guard<std::mutex> g(T.mu);
    for (int k = 0; k < SB_K_COUNT; ++k) {
        for (auto& p : T.ev[k]) {
            hipEventDestroy(p.first);
            hipEventDestroy(p.second);
        }
        T.ev[k].clear();
        for (auto e : T.open[k]) hipEventDestroy(e);
        T.open[k].clear();
    }
    return SB_OK;
}

// ------------------------------------------------------------------ op-level entry points
extern "C" int sb_op_gemm(int32_t dtype, int32_t epilogue, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda,
                          const void* W, int64_t ldw, const void* bias, void* C, int64_t ldc, int32_t out_f32, int32_t F,
                          void* stream) {
    if (dtype != SB_F32 && dtype != SB_BF16) return fail(SB_ERR_INVALID, "unknown dtype");
    GemmArgs a{};
    a.M = M;
    a.N = N;
    a.K = K;
    a.A = A;
    a.lda = lda;
    a.W = W;
    a.ldw = ldw;
    a.bias = bias;
    a.C = C;
    a.ldc = ldc;
    a.out_f32 = out_f32;
    a.F = F;
    return launch_gemm(dtype, epilogue, a, (hipStream_t)stream);
}

extern "C" int sb_op_norm(int32_t dtype, int32_t kind, int32_t rows, int32_t H, const float* x, const int32_t* row_map,
                          const void* g, const void* b, float eps, void* out, void* stream) {
    if (dtype != SB_F32 && dtype != SB_BF16) return fail(SB_ERR_INVALID, "unknown dtype");
    if (!x || !g || !out) return fail(SB_ERR_INVALID, "sb_op_norm: NULL argument");
    return launch_norm(dtype, kind, rows, H, x, row_map, g, b, eps, out, (hipStream_t)stream);
}

extern "C" int sb_op_rope_append(const sb_model_dims* dims, const sb_ragged* rg, const sb_kv* kv, int32_t layer, void* qkv,
                                 void* stream) {
    int st = validate_dims(dims);
    if (st) return st;
    void *kp, *vp;
    if ((st = sb_kv_layer_ptrs(kv, layer, &kp, &vp))) return st;
    return launch_rope_append(dims, rg, qkv, kp, vp, kv->arena_slots, (hipStream_t)stream);
}

extern "C" int sb_op_attention(const sb_model_dims* dims, const sb_ragged* rg, const sb_kv* kv, int32_t layer,
                               const void* qkv, void* o, void* workspace, size_t ws_bytes, void* stream) {
    int st = validate_dims(dims);
    if (st) return st;
    if (!rg || !kv || !qkv || !o) return fail(SB_ERR_INVALID, "sb_op_attention: NULL argument");
    size_t need = (size_t)rg->n_partials * 16 * (dims->head_dim + 2) * 4;
    if (rg->n_partials > 0 && (!workspace || ws_bytes < need)) return fail(SB_ERR_WORKSPACE, "attention partials need %zu bytes", need);
    void *kp, *vp;
    if ((st = sb_kv_layer_ptrs(kv, layer, &kp, &vp))) return st;
    float* po = (float*)workspace;
    float* pm = po ? po + (size_t)rg->n_partials * 16 * dims->head_dim : nullptr;
    return launch_attention(dims, rg, kp, vp, kv->arena_slots, qkv, o, po, pm, (hipStream_t)stream);
}

extern "C" int sb_op_argmax(int32_t rows, int32_t V, const float* logits, int32_t* out, void* stream) {
    if (!logits || !out || V <= 0) return fail(SB_ERR_INVALID, "sb_op_argmax: bad argument");
    return launch_argmax(rows, V, logits, out, (hipStream_t)stream);
}
