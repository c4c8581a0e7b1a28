// Per-request attention over the ragged batch in ONE launch.
//
// Orca runs attention request by request -- each request's queries attend only
// to that request's own K/V history -- and fuses the per-request attention
// into a single kernel by concatenating the requests' thread blocks
// ("CS349D Lecture 2", section 4.2; "连续批处理完全拆解", Figure 5).  Here the
// host builds a work list; every workgroup takes one item (a request, a K/V
// head, a tile of (token, query-head) rows and a key range), so prefills,
// decodes and prefill chunks share the launch.  Split / Merge are offsets:
// queries are read at their rows of the flattened qkv tensor and outputs are
// written to the same rows of o.
//
// Math per row (token j of request i, query head h): causal softmax over the
// request's keys 0..ctx_i + j of q.k / sqrt(d), times V.  Scores and the
// running max / sum live in fp32 (log2 domain).
//
// Tiling (CDNA4, 64-wide waves): S^T = K Q^T and O^T = V^T P^T, so that a
// query row's scores and outputs sit in the same lanes for both products and
// the softmax rescale needs no cross-lane moves.  The keys of a chunk are
// ordered so the S^T accumulators are directly the bf16 P^T operand; P is
// fed as a hi + lo pair of bf16 values (two MFMAs), which keeps P.V at about
// fp32 accuracy.
//   MODE_RUNS (<= 16 rows per request and K/V head: decodes, small chunks;
//     16x16x32 MFMAs, a row in lane % 16):
//     the 4 waves take interleaved 32-key chunks of a run of 512-key units;
//     K/V go straight from HBM into MFMA operand registers (16-byte loads,
//     the next chunk's loads in flight while the current one computes, also
//     across unit boundaries).  At the end of each unit the 4 wave states
//     merge through LDS.  A run that covers all of its request's units folds
//     the unit states in unit order itself; otherwise each unit leaves a
//     partial state, merged by attn_combine in unit order with the same
//     two-state merge, so the result does not depend on the rest of the batch.
//   MODE_ROWS (prefill tiles of 64 or 128 rows; 32x32x16 MFMAs): each wave
//     owns one 32-column block of rows (16 or 32 of them real); the workgroup
//     copies 64-key K/V tiles global -> LDS directly, the next tile in flight
//     while a tile computes, so the 4 waves share every K/V byte.  A row's
//     reference max moves only when a chunk's max exceeds it by more than
//     kLazyLog2, so the output accumulators are rarely rescaled.
#include <cfloat>
#include <mutex>
#include <type_traits>

#include "sb_device.h"
#include "sb_ops.h"

namespace sb {
namespace {

constexpr float kNegInf = -INFINITY;

struct AttnArgs {
    const void* qkv;
    long long qkv_stride;     // elements per row of qkv
    void* out;                // o [T, nq*d]
    long long out_stride;
    const void* K;            // layer plane base of K: [nkv][arena][d]
    const void* V;            // layer plane base of V: [nkv][arena/8][d][8]
    long long arena;
    const int* cu;
    const int* ctx;
    const int* tok_slot;
    const int* items;         // work items, one per workgroup
    float* part_o;            // [n_part][16][d]
    float* part_ml;           // [n_part][16][2]
    int nq, nkv, G;
    float scale_log2;         // log2(e) / sqrt(d)
};

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Probabilities of one chunk (8 per lane, finite, in [0, 1]) as the P^T operand of
// two MFMAs: hi = bf16(p) and lo = bf16(p - hi) (p - hi is exact in fp32), so P.V
// keeps about 16 significant bits of p.  Conversions round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ void split_p(const float (&p)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pack_bf16x2(p[2 * i], p[2 * i + 1]);
        l[i] = pack_bf16x2(p[2 * i] - __uint_as_float(h[i] << 16), p[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// The value of lane l ^ 32 (v_permlane32_swap: lanes 32..63 of the first operand trade places with
// lanes 0..31 of the second; with both operands v, the two results hold v of lanes 0..31 and of
// lanes 32..63, each in every lane).
__device__ __forceinline__ float swap32(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// values i0 .. i0 + 7 of a 32x32 MFMA accumulator as a hi + lo pair of bf16 operands (as split_p)
__device__ __forceinline__ void split_p8(const f32x16& p, int i0, bf16x8& hi, bf16x8& lo) {
    u32x4 hh, ll;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = p[i0 + 2 * i], b = p[i0 + 2 * i + 1];
        hh[i] = pack_bf16x2(a, b);
        ll[i] = pack_bf16x2(a - __uint_as_float(hh[i] << 16), b - __uint_as_float(hh[i] & 0xffff0000u));
    }
    hi = __builtin_bit_cast(bf16x8, hh);
    lo = __builtin_bit_cast(bf16x8, ll);
}

// Swizzle of the staged K tile of a prefill tile: the 16-byte piece p of local row r sits at position
// p ^ kt_swz(r).  The 16 lanes of a quarter-wave read 16 rows at one piece index; their positions then
// spread over all 64 banks.
template <int D>
__device__ __forceinline__ int kt_swz(int row) {
    constexpr int SH = D >= 128 ? 0 : (D == 64 ? 1 : 2);
    return (row >> SH) & (D / 8 - 1);
}

// A prefill row's reference max moves only when a chunk's max exceeds it by more than this (log2 units).
constexpr float kLazyLog2 = 8.f;

// o *= alpha, skipped when no row of the wave changed its max (alpha == 1 exactly)
template <int N>
__device__ __forceinline__ void rescale(f32x4 (&o)[N], float alpha) {
    if (__ballot(alpha != 1.f) == 0) return;
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] *= alpha;
}

// One wave's online-softmax state for its 16 rows (row = lane % 16).
template <int D>
struct WaveState {
    f32x4 o[D / 16];          // O^T accumulators: dims 16*db + 4*(lane/16) + r
    float m;                  // running max (log2 units), same in the 4 lanes of a row
    float l;                  // this lane's share of the running sum
};

template <int D>
__device__ __forceinline__ void state_init(WaveState<D>& s) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) s.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    s.m = kNegInf;
    s.l = 0.f;
}

// Apply one chunk's scores p_raw (8 values of this lane: keys of the chunk for
// row lane%16, already masked to -inf) to the state: returns the probabilities
// (to feed the P.V product) and rescales the accumulators.
__device__ __forceinline__ void softmax_chunk(float (&sc)[8], float& m, float& l, float& alpha) {
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    if (mn == kNegInf) {                 // nothing visible yet for this row
        alpha = 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[i] = 0.f;
        return;
    }
    // the hardware exp2 directly: arguments are <= 0, so results only differ from the library's below
    // 2^-126, where a probability adds nothing to the sums
    alpha = __builtin_amdgcn_exp2f(m - mn);       // m == -inf -> 0
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        sc[i] = __builtin_amdgcn_exp2f(sc[i] - mn);   // -inf -> 0
        sum += sc[i];
    }
    l = l * alpha + sum;
    m = mn;
}

// ------------------------------------------------------------------ bf16 chunk
// Keys of a 32-key chunk starting at key cb: S^T block b covers local keys
// 8*(m/4) + 4*b + (m%4) for MFMA row m, so that lane (g = lane/16) ends up
// with keys 8g..8g+7 -- exactly the P^T operand layout of the 16x16x32 MFMA.
// K/V registers of one 32-key chunk for the direct-from-HBM path (MODE_RUNS):
// K operands of the two S^T blocks and V^T operands of every 16-dim block.
template <int D>
struct ChunkRegs {
    u32x4 k[2][D / 32];
    u32x4 v[D / 16];
};

template <int D>
__device__ __forceinline__ void load_chunk_bf16(ChunkRegs<D>& r, const uint16_t* Kp, const uint16_t* Vp,
                                                long long kslot0, int cb, int key_end, int lane) {
    const int lr = lane & 15, g = lane >> 4;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int kk = min(cb + 8 * (lr >> 2) + 4 * b + (lr & 3), key_end - 1);   // clamp: masked later
#pragma unroll
        for (int s = 0; s < D / 32; ++s) r.k[b][s] = *(const u32x4*)(Kp + (kslot0 + kk) * D + s * 32 + g * 8);
    }
    const long long blk = (kslot0 + min(cb + 8 * g, key_end - 1)) >> 3;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) r.v[db] = *(const u32x4*)(Vp + (blk * D + db * 16 + lr) * 8);
}

template <int D>
__device__ __forceinline__ void compute_chunk_bf16(const AttnArgs& a, WaveState<D>& st, const bf16x8 (&qf)[D / 32],
                                                   const ChunkRegs<D>& r, int cb, int key_end, int row_limit,
                                                   int all_visible, int lane) {
    const int lr = lane & 15, g = lane >> 4;
    (void)lr;
    float sc[8];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k[b][s]), qf[s], acc, 0, 0, 0);
        if (cb + 32 <= all_visible) {
#pragma unroll
            for (int q = 0; q < 4; ++q) sc[4 * b + q] = acc[q] * a.scale_log2;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = cb + 8 * g + 4 * b + q;
                sc[4 * b + q] = (k < key_end && k < row_limit) ? acc[q] * a.scale_log2 : kNegInf;
            }
        }
    }
    float alpha;
    softmax_chunk(sc, st.m, st.l, alpha);
    rescale(st.o, alpha);
    bf16x8 ph, pl;
    split_p(sc, ph, pl);
    const int k8 = cb + 8 * g;
    const bool tail = k8 + 8 > key_end, any = k8 < key_end;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
        u32x4 vraw = r.v[db];
        if (tail) {
            union { u32x4 v; uint16_t h[8]; } vv;
            vv.v = vraw;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (!any || k8 + i >= key_end) vv.h[i] = 0;
            vraw = vv.v;
        }
        const bf16x8 vv8 = __builtin_bit_cast(bf16x8, vraw);
        st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv8, ph, st.o[db], 0, 0, 0);
        st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv8, pl, st.o[db], 0, 0, 0);
    }
}

// ------------------------------------------------------------------ fp32 chunk
// 16x16x4 fp32 MFMA: S^T block b covers keys cb + 16b + (lane%16) as MFMA rows;
// lane (g, r) gets keys cb + 16b + 4g + i.  P.V runs one 4-key step per (b, i).
template <int D>
__device__ __forceinline__ void chunk_f32(const AttnArgs& a, WaveState<D>& st, const float (&qf)[D / 4],
                                          const float* Kp, const float* Vp, long long kslot0, int cb,
                                          int key_end, int row_limit, int lane) {
    const int lr = lane & 15, g = lane >> 4;
    float sc[8];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int key = cb + 16 * b + lr;
        const int kk = min(key, key_end - 1);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < D / 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Kp[(kslot0 + kk) * D + 4 * s + g], qf[s], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int k = cb + 16 * b + 4 * g + r;
            sc[4 * b + r] = (k < key_end && k < row_limit) ? acc[r] * a.scale_log2 : kNegInf;
        }
    }
    float alpha;
    softmax_chunk(sc, st.m, st.l, alpha);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) st.o[i] *= alpha;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = cb + 16 * b + 4 * g + r;
            const bool ok = key < key_end;
            const long long slot = kslot0 + min(key, key_end - 1);
#pragma unroll
            for (int db = 0; db < D / 16; ++db) {
                float v = Vp[((slot >> 3) * D + db * 16 + lr) * 8 + (slot & 7)];
                v = ok ? v : 0.f;
                st.o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, sc[4 * b + r], st.o[db], 0, 0, 0);
            }
        }
}

// Softmax state of one row over some keys: running max m (log2 units), sum l
// and unnormalised output o over N dims.  merge2 folds state b into state a;
// requests whose keys span several units merge their units' states with it in
// unit order, inside the workgroup or in attn_combine -- the same operations
// either way, so the result never depends on where the merge ran.
__device__ __forceinline__ void merge_weights(float ma, float mb, float& M, float& wa, float& wb) {
    M = fmaxf(ma, mb);
    wa = (ma == kNegInf) ? 0.f : exp2f(ma - M);
    wb = (mb == kNegInf) ? 0.f : exp2f(mb - M);
}
__device__ __forceinline__ float merge_val(float a, float wa, float b, float wb) { return fmaf(a, wa, b * wb); }

// Per thread of a MODE_RUNS workgroup: row r = tid / 16, dims d0 .. d0 + DPT of that row.
template <int D>
struct RowState {
    static constexpr int DPT = D * 16 / 256;
    float m, l, o[DPT];
};

// Merge the four waves' states of one unit through LDS (fixed wave order) into
// this thread's (row, dims) share u.  Called by all 256 threads; leaves every
// wave's state reset for the next unit.
template <int D>
__device__ __forceinline__ void merge_unit(WaveState<D>& st, char* smem, RowState<D>& u) {
    constexpr int DPT = RowState<D>::DPT;
    float (*red_o)[16][D + 1] = (float (*)[16][D + 1])smem;
    float (*red_m)[16] = (float (*)[16])(smem + kWaves * 16 * (D + 1) * 4);
    float (*red_l)[16] = (float (*)[16])(smem + (kWaves * 16 * (D + 1) + kWaves * 16) * 4);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
    float l = st.l;                                  // this wave's row sum over the 4 lanes of the row
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) red_o[wave][lr][db * 16 + 4 * g + r] = st.o[db][r];
    if (g == 0) {
        red_m[wave][lr] = st.m;
        red_l[wave][lr] = l;
    }
    state_init(st);
    __syncthreads();
    const int r = tid / (256 / 16);
    const int d0 = (tid % (256 / 16)) * DPT;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][r]);
    float wts[kWaves], L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        wts[w] = (red_m[w][r] == kNegInf) ? 0.f : exp2f(red_m[w][r] - M);
        L = fmaf(red_l[w][r], wts[w], L);
    }
    u.m = M;
    u.l = L;
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) o = fmaf(red_o[w][r][d0 + e], wts[w], o);
        u.o[e] = o;
    }
    __syncthreads();                                 // LDS free for the next unit
}

template <int DT, int D>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
    using T = typename Store<DT>::T;
    constexpr int KT = 64;                                   // keys per LDS stage (MODE_ROWS)
    // MODE_ROWS stages K/V tiles; MODE_RUNS merges wave states: one workgroup uses only one of the two,
    // so they share the LDS allocation.  A MODE_ROWS stage holds a K tile [KT][D] then the KT / 8 V
    // blocks [D][8] of the same keys.
    constexpr int ROWS_NS = 2;                               // stages of the copy ring
    constexpr int ROWS_STAGE = 2 * KT * D;                   // elements per stage
    constexpr int ROWS_KI = KT * D * 2 / 1024;               // copy instructions of a K tile (= of a V tile)
    constexpr int ROWS_PERW = 2 * ROWS_KI / kWaves;          // per wave per stage
    static_assert(DT != SB_BF16 || ROWS_PERW * kWaves == 2 * ROWS_KI, "copies must split evenly over the waves");
    static_assert(ROWS_NS - 2 <= 2, "the wait ladder covers at most two tiles in flight");
    constexpr int BYTES_ROWS = (DT == SB_BF16) ? ROWS_NS * ROWS_STAGE * 2 : 0;
    constexpr int BYTES_RED = (kWaves * 16 * (D + 1) + 2 * kWaves * 16) * 4;
    __shared__ __attribute__((aligned(1024))) char smem[BYTES_ROWS > BYTES_RED ? BYTES_ROWS : BYTES_RED];
    const uint16_t* smem_u16 = (const uint16_t*)smem;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, g = lane >> 4;
    const int* it = a.items + (long long)blockIdx.x * kItemInts;
    const int req = it[ITEM_REQ], kvh = it[ITEM_KVH], mode = it[ITEM_MODE];
    const int row0 = it[ITEM_ROW0], nrows = it[ITEM_NROWS];
    const int kb = it[ITEM_KB], ke = it[ITEM_KE], part0 = it[ITEM_PART];
    if (nrows == 0) return;                      // an empty item (padding of the dispatch order)
    const int tok0 = it[ITEM_TOK0], ctx = it[ITEM_CTX];
    const long long kslot0 = it[ITEM_SLOT0];                      // slot of key 0 of this request
    const T* Kp = (const T*)a.K + (long long)kvh * a.arena * D;
    const T* Vp = (const T*)a.V + (long long)kvh * a.arena * D;

    // rows of this wave: (token, head-in-group), token-major
    const int wrow0 = row0 + (mode == MODE_ROWS ? wave * 16 : 0);
    const int row = wrow0 + lr;
    const bool row_ok = row < row0 + nrows;
    const int tok = row_ok ? row / a.G : 0;
    const int head = kvh * a.G + (row_ok ? row % a.G : 0);
    const int row_limit = row_ok ? ctx + tok + 1 : 0;             // keys 0..ctx+tok are visible
    // keys below this are visible to every row of the wave (its first row has the fewest)
    const int all_visible = min(ke, ctx + wrow0 / a.G + 1);
    const T* qrow = (const T*)a.qkv + (long long)(tok0 + tok) * a.qkv_stride + (long long)head * D;

    WaveState<D> st;
    state_init(st);

    if (mode == MODE_RUNS) {
        // Wave w takes chunks w, w + 4, ... of every unit; the chunk after a wave's last one in a unit
        // is its first one in the next unit, so the loads run ahead across unit boundaries.
        // End of each unit: merge the waves' states; then either store the unit's partial state
        // (the request's units are spread over several runs: part0 >= 0) or fold it into this
        // thread's running state of the request (the run covers all of the request's units).
        constexpr int DPT = RowState<D>::DPT;
        const int rr = tid / (256 / 16), d0 = (tid % (256 / 16)) * DPT;
        RowState<D> acc;
        auto end_unit = [&](int u0) {
            RowState<D> u;
            merge_unit<D>(st, smem, u);
            if (part0 >= 0) {
                if (rr < nrows) {
                    const long long p = part0 + (u0 - kb) / kUnitKeys;
                    float* po = a.part_o + (p * 16 + rr) * D + d0;
#pragma unroll
                    for (int e = 0; e < DPT; ++e) po[e] = u.o[e];
                    if (d0 == 0) {
                        a.part_ml[(p * 16 + rr) * 2 + 0] = u.m;
                        a.part_ml[(p * 16 + rr) * 2 + 1] = u.l;
                    }
                }
            } else if (u0 == kb) {
                acc = u;
            } else {
                float M, wa, wb;
                merge_weights(acc.m, u.m, M, wa, wb);
                acc.l = merge_val(acc.l, wa, u.l, wb);
#pragma unroll
                for (int e = 0; e < DPT; ++e) acc.o[e] = merge_val(acc.o[e], wa, u.o[e], wb);
                acc.m = M;
            }
        };
        auto next_chunk = [&](int cb) {
            const int u0 = cb - (cb - kb) % kUnitKeys;
            const int n = cb + 32 * kWaves;
            return n < min(u0 + kUnitKeys, ke) ? n : u0 + kUnitKeys + 32 * wave;
        };
        if constexpr (DT == SB_BF16) {
            bf16x8 qf[D / 32];
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                u32x4 v = row_ok ? *(const u32x4*)(qrow + s * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
                qf[s] = __builtin_bit_cast(bf16x8, v);
            }
            const uint16_t* Kb = (const uint16_t*)Kp;
            const uint16_t* Vb = (const uint16_t*)Vp;
            ChunkRegs<D> cur, nxt;
            int cb = kb + 32 * wave;                       // this wave's current chunk (>= ke: none left)
            load_chunk_bf16<D>(cur, Kb, Vb, kslot0, min(cb, ke - 1), ke, lane);
            for (int u0 = kb; u0 < ke; u0 += kUnitKeys) {
                const int ue = min(u0 + kUnitKeys, ke);
                while (cb < ue) {
                    const int nb = next_chunk(cb);
                    // issued whether or not a next chunk exists (then it re-reads this one): an
                    // unconditional load lets the compiler keep it in flight during the compute
                    load_chunk_bf16<D>(nxt, Kb, Vb, kslot0, nb < ke ? nb : cb, ke, lane);
                    compute_chunk_bf16<D>(a, st, qf, cur, cb, ke, row_limit, all_visible, lane);
                    cur = nxt;
                    cb = nb;
                }
                end_unit(u0);
            }
        } else {
            float qf[D / 4];
#pragma unroll
            for (int s = 0; s < D / 4; ++s) qf[s] = row_ok ? ((const float*)qrow)[4 * s + g] : 0.f;
            for (int u0 = kb; u0 < ke; u0 += kUnitKeys) {
                const int ue = min(u0 + kUnitKeys, ke);
                for (int cb = u0 + 32 * wave; cb < ue; cb += 32 * kWaves)
                    chunk_f32<D>(a, st, qf, (const float*)Kp, (const float*)Vp, kslot0, cb, ke, row_limit, lane);
                end_unit(u0);
            }
        }
        // a run that covers all of its request's units: normalise the merged state
        if (part0 < 0 && rr < nrows) {
            const int tk = rr / a.G, hd = kvh * a.G + rr % a.G;
            T* orow = (T*)a.out + (long long)(tok0 + tk) * a.out_stride + (long long)hd * D + d0;
#pragma unroll
            for (int e = 0; e < DPT; ++e) Store<DT>::st(orow + e, acc.o[e] / acc.l);
        }
        return;
    }

    // MODE_ROWS (bf16): a tile of up to 64 x rbn rows; wave w owns rows row0 + 16 rbn w + c for the
    // columns c < 16 rbn of one 32-column block (lane c and lane c + 32 share row c; other columns are
    // padding: q = 0, every key visible, never stored).  KT-key K/V tiles are copied global -> LDS
    // directly (global_load_lds_dwordx4) into a ring of NS stages, one tile ahead of the one being
    // computed.  Per tile and wave: S^T = K Q^T as two 32-key blocks of 32x32x16 MFMAs, the softmax
    // update in registers, then O^T += V^T P^T as 16-key steps.
    if constexpr (DT == SB_BF16) {
        constexpr int NP = D / 8;                      // 16-byte pieces of a K row
        const int rbn = it[ITEM_RB];
        const int c = lane & 31, h = lane >> 5;
        const int wr0 = row0 + wave * 16 * rbn;        // first row of the wave
        const int wend = min(wr0 + 16 * rbn, row0 + nrows);
        const int rrow = wr0 + c;
        const bool ok = c < 16 * rbn && rrow < wend;
        const int rtok = ok ? rrow / a.G : 0;
        const int rhead = kvh * a.G + (ok ? rrow % a.G : 0);
        const int rl = ok ? ctx + rtok + 1 : ke;      // keys below rl are visible to this column
        // keys below all_vis are visible to every row of the wave (its first row sees the fewest); keys at
        // or past wmax to none
        const int all_vis = min(ke, ctx + wr0 / a.G + 1);
        const int wmax = wr0 < wend ? min(ke, ctx + (wend - 1) / a.G + 1) : 0;
        // S^T row m of a 32-key block holds local key pi(m) (bits 2 and 3 of m swapped): the accumulator
        // values of a lane are then, eight at a time, the P^T operand of one 16-key step of O^T += V^T P^T
        const int pic = (c & ~12) | ((c & 4) << 1) | ((c & 8) >> 1);
        bf16x8 qf[D / 16];                             // Q^T operand: dims 16 s + 8 h .. + 8 of row c
        {
            const T* q = (const T*)a.qkv + (long long)(tok0 + rtok) * a.qkv_stride + (long long)rhead * D;
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                u32x4 v = ok ? *(const u32x4*)(q + 16 * s + 8 * h) : u32x4{0u, 0u, 0u, 0u};
                qf[s] = __builtin_bit_cast(bf16x8, v);
            }
        }
        f32x16 oacc[D / 32];                           // O^T: dims 32 db + 8 (i / 4) + 4 h + i % 4 of row c
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
        float m = kNegInf, l = 0.f;                    // reference max (log2 units) and this lane's sum
        // the q loads are the only loads the compiler sees: complete them before any copy is in flight,
        // so that no wait it inserts later also waits for the copies
        wait_vmcnt<0>();
        const int ntiles = (ke - kb + KT - 1) / KT;
        const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
        const long long vlast = (kslot0 + ke - 1) >> 3;
        // copy instruction q of the tile starting at key k0 into stage `stage`: K rows first (R rows of D
        // elements per instruction; lane L fills position L % NP of row L / NP with the source piece that
        // belongs there, (L % NP) ^ kt_swz(row)), then the V blocks (8 keys x D dims each, as in the arena;
        // a block of D = 32 is half an instruction).  Keys at or past ke read key ke - 1 (K) or the block
        // holding it (V): finite values, masked in the compute.
        auto copy = [&](int stage, int k0, int q) {
            const uint32_t sbase = lds0 + (uint32_t)(stage * ROWS_STAGE * 2);
            if (q < ROWS_KI) {
                constexpr int R = 1024 / (D * 2);
                const int row = q * R + lane / NP, p = lane % NP;
                const long long slot = kslot0 + min(k0 + row, ke - 1);
                dma16((const uint16_t*)Kp + slot * D + ((p ^ kt_swz<D>(row)) << 3), sbase + q * 1024);
            } else {
                const int j = q - ROWS_KI;
                if constexpr (D >= 64) {
                    constexpr int PB = D * 16 / 1024;          // instructions per V block
                    const int vb = j / PB, hh = j % PB;
                    const long long blk = min(((kslot0 + k0) >> 3) + vb, vlast);
                    dma16((const uint16_t*)Vp + blk * D * 8 + hh * 512 + lane * 8, sbase + KT * D * 2 + j * 1024);
                } else {
                    const int vb = 2 * j + lane / 32;           // two 512-byte blocks per instruction
                    const long long blk = min(((kslot0 + k0) >> 3) + vb, vlast);
                    dma16((const uint16_t*)Vp + blk * D * 8 + (lane % 32) * 8, sbase + KT * D * 2 + j * 1024);
                }
            }
        };
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);      // wave-uniform, for the copies' LDS base
        // Copies of a tile whose keys all lie below ke need no clamping: this wave's copy i then reads
        // cbase + (kslot0 + k0) D + src_off[i] (waves 0 and 1 copy K rows, waves 2 and 3 V blocks).
        const uint16_t* cbase = (const uint16_t*)(wave_u * ROWS_PERW < ROWS_KI ? Kp : Vp);
        int src_off[ROWS_PERW];
#pragma unroll
        for (int i = 0; i < ROWS_PERW; ++i) {
            const int q = wave_u * ROWS_PERW + i;
            if (q < ROWS_KI) {
                constexpr int R = 1024 / (D * 2);
                const int row = q * R + lane / NP, p = lane % NP;
                src_off[i] = row * D + ((p ^ kt_swz<D>(row)) << 3);
            } else if constexpr (D >= 64) {
                constexpr int PB = D * 16 / 1024;
                const int j = q - ROWS_KI;
                src_off[i] = (j / PB) * D * 8 + (j % PB) * 512 + lane * 8;
            } else {
                const int j = q - ROWS_KI;
                src_off[i] = (2 * j + lane / 32) * D * 8 + (lane % 32) * 8;
            }
        }
        auto issue = [&](int stage, int t) {
            const int k0 = kb + t * KT;
            if (k0 + KT <= ke) {
                const uint16_t* src = cbase + (kslot0 + k0) * D;
                const uint32_t sbase = lds0 + (uint32_t)(stage * ROWS_STAGE * 2) + (uint32_t)(wave_u * ROWS_PERW * 1024);
#pragma unroll
                for (int i = 0; i < ROWS_PERW; ++i) dma16(src + src_off[i], sbase + i * 1024);
            } else {
#pragma unroll
                for (int i = 0; i < ROWS_PERW; ++i) copy(stage, k0, wave_u * ROWS_PERW + i);
            }
        };
        auto compute = [&](int t, int stage) {
            const int cb = kb + t * KT;
            if (cb >= wmax) return;                      // no row of this wave sees these keys
            const uint16_t* lk = smem_u16 + stage * ROWS_STAGE;
            const uint16_t* lv = lk + KT * D;
            f32x16 sacc[2];
            // the MFMA phases (S^T and P.V) issue at raised wave priority, so that while one wave feeds the matrix
            // unit the other wave on the SIMD fills the gaps with its softmax (175B-shaped prompts: -2%)
            __builtin_amdgcn_s_setprio(1);
            {
                bf16x8 kf[2][D / 16];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int r = 32 * b + pic;
                    const int sw = kt_swz<D>(r);
#pragma unroll
                    for (int s = 0; s < D / 16; ++s) kf[b][s] = *(const bf16x8*)(lk + r * D + (((2 * s + h) ^ sw) << 3));
#pragma unroll
                    for (int i = 0; i < 16; ++i) sacc[b][i] = 0.f;
                }
#pragma unroll
                for (int s = 0; s < D / 16; ++s)
#pragma unroll
                    for (int b = 0; b < 2; ++b) sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[b][s], qf[s], sacc[b], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
            // value i of block b is the score of key cb + 32 b + 16 (i / 8) + 8 h + i % 8
            if (cb + KT > all_vis) {
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (cb + 32 * b + 16 * (i / 8) + 8 * h + (i % 8) >= rl) sacc[b][i] = kNegInf;
            }
            float mx = sacc[0][0];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[b][i]);
            mx = fmaxf(mx, swap32(mx));                  // the row's other 32 keys sit in lane c ^ 32
            // lazy reference max: moved only when the chunk's max exceeds it by more than kLazyLog2, so the
            // accumulators are rarely rescaled; probabilities stay below 2^kLazyLog2
            const float mxs = mx * a.scale_log2;
            const bool up = mxs > m + kLazyLog2;
            const float mn = up ? mxs : m;
            const float alpha = up ? __builtin_amdgcn_exp2f(m - mn) : 1.f;   // m == -inf -> 0
            m = mn;
            const float nm = (mn == kNegInf) ? 0.f : -mn;
            float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    sacc[b][i] = __builtin_amdgcn_exp2f(fmaf(sacc[b][i], a.scale_log2, nm));   // -inf -> 0
                    ps[i % 4] += sacc[b][i];
                }
            const float sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
            l = l * alpha + sum;
            if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
            }
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int j = 0; j < KT / 16; ++j) {
                bf16x8 ph, pl;
                split_p8(sacc[j / 2], 8 * (j % 2), ph, pl);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    // V^T operand: keys cb + 16 j + 8 h .. + 8 at dim 32 db + c, 16 contiguous bytes of a block
                    const bf16x8 vv = *(const bf16x8*)(lv + (2 * j + h) * 8 * D + (32 * db + c) * 8);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, ph, oacc[db], 0, 0, 0);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pl, oacc[db], 0, 0, 0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        };
        // ring: tile t in stage t % NS; step t waits for its own copies of tile t, then the barrier (every
        // wave's copies of tile t landed; every wave finished tile t - 1), then issues tile t + NS - 1 into
        // the stage tile t - 1 used, then computes tile t
#pragma unroll
        for (int t = 0; t < ROWS_NS - 1; ++t)
            if (t < ntiles) issue(t, t);
        for (int t = 0; t < ntiles; ++t) {
            const int later = min(ROWS_NS - 2, ntiles - 1 - t);     // tiles issued after t, still in flight
            if (later >= 2) wait_vmcnt<2 * ROWS_PERW>();
            else if (later == 1) wait_vmcnt<ROWS_PERW>();
            else wait_vmcnt<0>();
            lds_barrier();
            if (t + ROWS_NS - 1 < ntiles) issue((t + ROWS_NS - 1) % ROWS_NS, t + ROWS_NS - 1);
            if (t == ntiles - 1 && kb + (t + 1) * KT > ke) {
                // the last tile holds keys at or past ke: zero their V entries (a probability of 0 times
                // stale memory could be NaN); K rows there are copies of key ke - 1, masked in the scores
                // blocks of 8 keys [D][8]: the blocks past the one holding key ke - 1 as whole 16-byte rows,
                // that block's entries past ke - 1 with one masked rewrite of each of its D rows
                const int nvalid = ke - (kb + t * KT);
                uint16_t* lvw = (uint16_t*)smem + (t % ROWS_NS) * ROWS_STAGE + KT * D;
                const int vb0 = nvalid >> 3, e0 = nvalid & 7;
                const int zb = e0 ? vb0 + 1 : vb0;              // first block with no valid key
                for (int r = tid; r < (KT / 8 - zb) * D; r += 256) *(u32x4*)(lvw + (zb * D + r) * 8) = u32x4{0u, 0u, 0u, 0u};
                if (e0) {
                    for (int d = tid; d < D; d += 256) {
                        u32x4* row = (u32x4*)(lvw + (vb0 * D + d) * 8);
                        u32x4 v = *row;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] &= (2 * e < e0 ? 0xffffu : 0u) | (2 * e + 1 < e0 ? 0xffff0000u : 0u);
                        *row = v;
                    }
                }
                __syncthreads();
            }
            compute(t, t % ROWS_NS);
        }
        const float lt = l + swap32(l);                  // l of lane c plus that of lane c ^ 32 (the same in both lanes)
        if (ok) {
            const float inv = 1.f / lt;
            T* orow = (T*)a.out + (long long)(tok0 + rtok) * a.out_stride + (long long)rhead * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    u32x2 v;
                    v[0] = pack_bf16x2(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv);
                    v[1] = pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
                    *(u32x2*)(orow + 32 * db + 8 * g4 + 4 * h) = v;
                }
        }
        return;
    } else {
        float qf[D / 4];
#pragma unroll
        for (int s = 0; s < D / 4; ++s) qf[s] = row_ok ? ((const float*)qrow)[4 * s + g] : 0.f;
        for (int cb = kb; cb < ke; cb += 32)
            chunk_f32<D>(a, st, qf, (const float*)Kp, (const float*)Vp, kslot0, cb, ke, row_limit, lane);
    }

    // total row sum over the 4 lanes of the row
    float l = st.l;
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (!row_ok) return;
    const float inv = 1.f / l;
    T* orow = (T*)a.out + (long long)(tok0 + tok) * a.out_stride + (long long)head * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) Store<DT>::st(orow + db * 16 + 4 * g + r, st.o[db][r] * inv);
}

// Merge the unit partials of one (request, K/V head) tile, in unit order, with
// the same two-state merge the attention workgroups use for whole requests.
template <int DT, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, const int* groups) {
    using T = typename Store<DT>::T;
    const int* gp = groups + (long long)blockIdx.x * kGroupInts;
    const int req = gp[GRP_REQ], kvh = gp[GRP_KVH], row0 = gp[GRP_ROW0], nrows = gp[GRP_NROWS];
    const int p0 = gp[GRP_PART0], np = gp[GRP_NPARTS];
    const int tok0 = gp[GRP_TOK0];
    for (int idx = threadIdx.x; idx < 16 * D; idx += 256) {
        const int r = idx / D, e = idx % D;
        if (r >= nrows) break;
        const long long q0 = (long long)p0 * 16 + r;
        float m = a.part_ml[q0 * 2], l = a.part_ml[q0 * 2 + 1], o = a.part_o[q0 * D + e];
        for (int p = 1; p < np; ++p) {
            const long long q = (long long)(p0 + p) * 16 + r;
            float M, wa, wb;
            merge_weights(m, a.part_ml[q * 2], M, wa, wb);
            l = merge_val(l, wa, a.part_ml[q * 2 + 1], wb);
            o = merge_val(o, wa, a.part_o[q * D + e], wb);
            m = M;
        }
        const int rr = row0 + r, tk = rr / a.G, hd = kvh * a.G + rr % a.G;
        Store<DT>::st((T*)a.out + (long long)(tok0 + tk) * a.out_stride + (long long)hd * D + e, o / l);
    }
}

template <int DT, int D>
int launch_attn_d(const AttnArgs& a, int n_items, int n_groups, const int* groups, hipStream_t s) {
    if (n_items > 0) {
        TimedScope ts(SB_K_ATTN, s);
        hipLaunchKernelGGL((attn_kernel<DT, D>), dim3(n_items), dim3(256), 0, s, a);
        int st = check_launch("attention");
        if (st) return st;
    }
    if (n_groups > 0) {
        TimedScope ts(SB_K_ATTN_COMBINE, s);
        hipLaunchKernelGGL((attn_combine_kernel<DT, D>), dim3(n_groups), dim3(256), 0, s, a, groups);
        return check_launch("attention combine");
    }
    return SB_OK;
}

}  // namespace

int launch_attention(const sb_model_dims* dims, const sb_ragged* rg, const void* kplane, const void* vplane,
                     long long arena, const void* qkv, void* out, float* part_o, float* part_ml, hipStream_t s) {
    AttnArgs a{};
    const int D = dims->head_dim;
    a.qkv = qkv;
    a.qkv_stride = (long long)(dims->n_heads + 2 * dims->n_kv_heads) * D;
    a.out = out;
    a.out_stride = (long long)dims->n_heads * D;
    a.K = kplane;
    a.V = vplane;
    a.arena = arena;
    a.cu = rg->cu_seqlens;
    a.ctx = rg->ctx_lens;
    a.tok_slot = rg->tok_slot;
    a.items = rg->items;
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.nq = dims->n_heads;
    a.nkv = dims->n_kv_heads;
    a.G = dims->n_heads / dims->n_kv_heads;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    if (dims->dtype == SB_BF16) {
        switch (D) {
            case 32: return launch_attn_d<SB_BF16, 32>(a, rg->n_items, rg->n_groups, rg->groups, s);
            case 64: return launch_attn_d<SB_BF16, 64>(a, rg->n_items, rg->n_groups, rg->groups, s);
            case 128: return launch_attn_d<SB_BF16, 128>(a, rg->n_items, rg->n_groups, rg->groups, s);
        }
    } else {
        switch (D) {
            case 16: return launch_attn_d<SB_F32, 16>(a, rg->n_items, rg->n_groups, rg->groups, s);
            case 32: return launch_attn_d<SB_F32, 32>(a, rg->n_items, rg->n_groups, rg->groups, s);
            case 64: return launch_attn_d<SB_F32, 64>(a, rg->n_items, rg->n_groups, rg->groups, s);
            case 128: return launch_attn_d<SB_F32, 128>(a, rg->n_items, rg->n_groups, rg->groups, s);
        }
    }
    return fail(SB_ERR_INVALID, "attention: unsupported head_dim %d", D);
}

}  // namespace sb

// ------------------------------------------------------------------ allocation-free attention
// A variant of sb_op_attention whose unit partials live in a file-scope device array instead of a
// caller-provided workspace.  Host code must never pass `scratch` itself to a kernel: in host code
// the name is a stand-in, not a device address.  Its address on each device comes from
// hipGetSymbolAddress, taken once per device with that device current and kept in g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[SB_ATTN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (taken on the first call on that device).
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return sb::fail(SB_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return sb::fail(SB_ERR_DEVICE, "device %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return sb::fail(SB_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return SB_OK;
}
}  // namespace

extern "C" int sb_op_attention_noalloc(const sb_model_dims* dims, const sb_ragged* rg, const sb_kv* kv, int32_t layer,
                                       const void* qkv, void* o, void* stream) {
    int st = sb::validate_dims(dims);
    if (st) return st;
    if (!rg || !kv || !qkv || !o) return sb::fail(SB_ERR_INVALID, "sb_op_attention_noalloc: NULL argument");
    const size_t need = (size_t)rg->n_partials * 16 * (dims->head_dim + 2) * 4;
    if (need > (size_t)SB_ATTN_NOALLOC_SCRATCH_BYTES)
        return sb::fail(SB_ERR_WORKSPACE, "attention partials need %zu bytes, the static scratch holds %zu", need,
                        (size_t)SB_ATTN_NOALLOC_SCRATCH_BYTES);
    void *kp, *vp;
    if ((st = sb_kv_layer_ptrs(kv, layer, &kp, &vp))) return st;
    float* po = nullptr;
    float* pm = nullptr;
    if (rg->n_partials > 0) {
        void* base = nullptr;
        if ((st = scratch_address(&base))) return st;
        po = (float*)base;
        pm = po + (size_t)rg->n_partials * 16 * dims->head_dim;
    }
    return sb::launch_attention(dims, rg, kp, vp, kv->arena_slots, qkv, o, po, pm, (hipStream_t)stream);
}
