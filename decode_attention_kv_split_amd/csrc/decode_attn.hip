// gfx950 kernels and C ABI for split-KV decode attention over a growing KV cache.
//
// Method (page "MoA-Structured Decode Attention"): per query head, Step I scores every
// cached K row against q (eq. 1, K read row by row in its stored layout, no transpose),
// Step II takes a max-subtracted softmax of the scores (eq. 2) and Step III sums the V
// rows weighted by it (eq. 3). §5 appends one row per step at its row-major offset, §6
// lets every query head of a group select the group's KV rows instead of a copy.
//
// MI355X mapping (CDNA4, wave64):
//   * The cache rows of one (sequence, KV head) are cut into splits of `chunk` rows; one
//     256-thread workgroup handles one split for GT query heads of the group. The grid is
//     (splits at max_len, h_kv * g / GT, batch); splits past a sequence's end exit at once.
//   * Lanes span the head dimension (the page's coalescing criterion, §4: adjacent lanes
//     touch adjacent addresses): LPR lanes cover one row with one 8- or 16-byte load each,
//     so a wave loads 64 / LPR whole rows per instruction, fully coalesced.
//   * Each K and V row is loaded once into registers and used by all GT heads of the
//     group: KV bytes are read once per workgroup, not once per query head.
//   * The LPR partial dot products of a row are summed with DPP row permutes (no LDS).
//   * Softmax runs online in fp32 in the base-2 domain (scale * log2 e folded into the
//     score scale, v_exp_f32 for 2^x); each row group of a wave keeps its own running max,
//     sum and output, merged at the end of the split, then the four waves merge in LDS.
//   * Each split writes (max, sum, unnormalised output) per head; the combine kernel merges
//     splits by log-sum-exp weights. No atomics touch the output, so results are
//     deterministic run to run.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <algorithm>

#include "decode_attn.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;  // waves per split workgroup
constexpr int kBlock = kWave * kWaves;
constexpr int kUnroll = 4;  // row loads per lane per tile
constexpr int kCombineBlock = 256;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegBig = -3.0e38f;  // finite "minus infinity" for running maxima
constexpr size_t kHeaderBytes = 256;  // error word + padding at the workspace start

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ element traits
// kEpl elements per lane per row load; the load is kEpl * element-size bytes.
template <int KV> struct Kv;
template <> struct Kv<DA_F32> { static constexpr int kEsz = 4, kEpl = 4; using Vec = uint4; };
template <> struct Kv<DA_BF16> { static constexpr int kEsz = 2, kEpl = 8; using Vec = uint4; };
template <> struct Kv<DA_FP8_E4M3FN> { static constexpr int kEsz = 1, kEpl = 8; using Vec = uint2; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// OCP e4m3fn code -> fp32 for finite codes. The 7 magnitude bits shifted into an fp32's
// exponent/mantissa fields give 2^(e-127) * 1.mmm (or a subnormal m * 2^-129 when e = 0);
// multiplying by 2^120 rebiases to 2^(e-7) * 1.mmm and m * 2^-9 respectively, both exact.
// The NaN codes 0x7F / 0xFF are not produced by the quantiser and are not special-cased.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
    const float mag = __uint_as_float((c & 0x7Fu) << 20) * 0x1.0p120f;
    return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// Widen one lane's load into kEpl floats.
template <int KV>
__device__ __forceinline__ void widen(const typename Kv<KV>::Vec &v, float *f) {
    if constexpr (KV == DA_F32) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    } else if constexpr (KV == DA_BF16) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(w[i]); f[2 * i + 1] = bf16_hi(w[i]); }
    } else {
        const uint32_t w[2] = {v.x, v.y};
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = e4m3fn_to_f32((w[i / 4] >> (8 * (i % 4))) & 0xFFu);
    }
}

// ------------------------------------------------------------------ buffer loads
// Raw buffer loads: a 128-bit resource holds the base address and the number of valid
// bytes; a lane whose offset is at or past that count reads zeros without touching
// memory. Word 3 = 0x00020000 is the gfx9-family (incl. gfx950) default format.
// KV rows are streamed exactly once, so they are loaded with the non-temporal hint (cache
// policy bit 1, "nt"), which keeps them from displacing other lines; measured on MI355X it
// raises the split kernel's sustained read rate by 5-10 %.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kLoadNonTemporal = 2;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

template <typename Vec>
__device__ __forceinline__ Vec buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (sizeof(Vec) == 16) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kLoadNonTemporal);
        return Vec{x[0], x[1], x[2], x[3]};
    } else {
        const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kLoadNonTemporal);
        return Vec{x[0], x[1]};
    }
}

// ------------------------------------------------------------------ cross-lane sums
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of LPR consecutive lanes; every lane gets its group's sum.
// quad_perm [1,0,3,2] and [2,3,0,1] sum a quad; row_half_mirror pairs quads inside
// 8 lanes; row_mirror pairs halves inside a 16-lane row; 32 needs a cross-row swizzle.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (LPR >= 2) x += dpp<0xB1>(x);
    if constexpr (LPR >= 4) x += dpp<0x4E>(x);
    if constexpr (LPR >= 8) x += dpp<0x141>(x);
    if constexpr (LPR >= 16) x += dpp<0x140>(x);
    if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
    return x;
}

// ------------------------------------------------------------------ kernels
// Zeroes n words (the whole workspace: error word and partial results).
__global__ void workspace_init_kernel(int32_t *ws, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        ws[i] = 0;
}

// One workgroup per sequence: copy the h_kv new K rows and V rows into row lens[b] in
// 16-byte pieces, then (after every thread has read lens[b]) advance lens[b].
__global__ __launch_bounds__(256) void kv_append_kernel(
    char *__restrict__ kc, char *__restrict__ vc, int32_t *__restrict__ lens,
    const char *__restrict__ kn, const char *__restrict__ vn, int32_t *__restrict__ err,
    int h_kv, int cap, int row_k, int row_v) {
    const int b = blockIdx.x;
    const int L = lens[b];
    if (L < 0 || L >= cap) {
        if (threadIdx.x == 0 && err) atomicOr(err, DA_DEV_ERR_APPEND_FULL);
        return;
    }
    const int pk = row_k / 16, pv = row_v / 16;
    for (int i = threadIdx.x; i < h_kv * pk; i += blockDim.x) {
        const size_t slot = (size_t)b * h_kv + i / pk;
        const uint4 x = reinterpret_cast<const uint4 *>(kn + slot * row_k)[i % pk];
        reinterpret_cast<uint4 *>(kc + (slot * cap + L) * row_k)[i % pk] = x;
    }
    for (int i = threadIdx.x; i < h_kv * pv; i += blockDim.x) {
        const size_t slot = (size_t)b * h_kv + i / pv;
        const uint4 x = reinterpret_cast<const uint4 *>(vn + slot * row_v)[i % pv];
        reinterpret_cast<uint4 *>(vc + (slot * cap + L) * row_v)[i % pv] = x;
    }
    __syncthreads();
    if (threadIdx.x == 0) lens[b] = L + 1;
}

// Arguments of the split kernel (passed by value as one kernel argument).
struct SplitArgs {
    const void *q, *kc, *vc;
    const int32_t *lens;
    const float *kv_scales;   // [B, h_kv, 2] for fp8 caches, else unused
    float *part_ml, *part_o;  // per-split (max, sum) and unnormalised output rows
    float *out;               // decode_attn_run: output rows of single-split sequences
    int32_t *err;             // sticky device error word
    int h_q, h_kv, cap, chunk, n_splits, max_len;
    float qk_scale;           // scale * log2(e)
};

// One workgroup = one split of one (sequence, KV head) for GT query heads of its group.
// Every split writes part_ml[(b*h_q+h)*n_splits+split] = (max, sum) in the base-2 domain and
// part_o[...*D + d] = its unnormalised output row (times the V scale for fp8 caches);
// lse_combine_kernel merges them. With DIRECT (decode_attn_run) a sequence that fits one
// split writes its normalised output straight to out and the combine skips it.
template <int KV, int D, int GT, bool DIRECT>
__global__ __launch_bounds__(kBlock) void split_kv_attn_kernel(const SplitArgs a) {
    using T = Kv<KV>;
    using Vec = typename T::Vec;
    constexpr int EPL = T::kEpl;
    constexpr int LPR = D / EPL;       // lanes per row
    constexpr int RPL = kWave / LPR;   // rows per wave load
    constexpr int TILE = kUnroll * RPL;  // rows per wave per iteration
    constexpr int STEP = TILE * kWaves;  // rows per workgroup per iteration
    const int h_q = a.h_q, h_kv = a.h_kv, chunk = a.chunk;

    const int split = blockIdx.x;
    const int g = h_q / h_kv;
    const int tiles = g / GT;
    const int kvh = blockIdx.y / tiles;
    const int h0 = kvh * g + (blockIdx.y % tiles) * GT;
    const int b = blockIdx.z;

    const int L = a.lens[b];
    if (L < 1 || L > a.max_len) return;  // flagged and zeroed by the combine
    const int nsplit_b = (L + chunk - 1) / chunk;  // splits this sequence really has
    const int r0 = split * chunk;
    if (r0 >= L) return;
    const int r1 = min(r0 + chunk, L);

    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int grp = lane / LPR, sub = lane % LPR;

    const size_t slot = (size_t)b * h_kv + kvh;
    constexpr uint32_t ROWB = D * T::kEsz;  // bytes per cache row
    // Resources cover rows [0, r1) of this (sequence, KV head): loads of rows past the
    // split's end return zeros (and are masked out of the softmax below).
    const size_t slot_bytes = (size_t)a.cap * ROWB;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const char *>(a.kc) + slot * slot_bytes, r1 * ROWB);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(static_cast<const char *>(a.vc) + slot * slot_bytes, r1 * ROWB);
    const uint32_t lane_off = grp * ROWB + sub * (uint32_t)sizeof(Vec);
    float vscale = 1.f, sc = a.qk_scale;
    if constexpr (KV == DA_FP8_E4M3FN) {
        sc *= a.kv_scales[slot * 2 + 0];
        vscale = a.kv_scales[slot * 2 + 1];
    }

    // This lane's slice of q for the GT heads: fp32 values, or packed bf16 pairs for the
    // bf16 dot instruction.
    float qf[GT][EPL];
    uint32_t qp[GT][EPL / 2];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        const size_t qoff = ((size_t)b * h_q + h0 + h) * D + sub * EPL;
        if constexpr (KV == DA_F32) {
            const float4 x = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.q) + qoff);
            qf[h][0] = x.x; qf[h][1] = x.y; qf[h][2] = x.z; qf[h][3] = x.w;
        } else {
            const uint4 x = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + qoff);
            if constexpr (KV == DA_BF16) {
                qp[h][0] = x.x; qp[h][1] = x.y; qp[h][2] = x.z; qp[h][3] = x.w;
            } else {
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) { qf[h][2 * i] = bf16_lo(w[i]); qf[h][2 * i + 1] = bf16_hi(w[i]); }
            }
        }
    }

    float m[GT], l[GT], o[GT][EPL];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        m[h] = kNegBig;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
    }

    // Steps I-III on one tile already in registers: scores for the GT heads, an online
    // softmax update of (m, l, o), then the weighted V rows.
    auto process = [&](const Vec (&kt)[kUnroll], const Vec (&vt)[kUnroll], int tbase) {
        float s[GT][kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool valid = tbase + u * RPL + grp < r1;
            float kf[EPL];
            if constexpr (KV != DA_BF16) widen<KV>(kt[u], kf);
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                float acc = 0.f;
                if constexpr (KV == DA_BF16) {
                    const uint32_t w[4] = {kt[u].x, kt[u].y, kt[u].z, kt[u].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]),
                                                              __builtin_bit_cast(bf16x2_t, qp[h][i]),
                                                              acc, false);
                } else {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc = fmaf(kf[e], qf[h][e], acc);
                }
                acc = group_sum<LPR>(acc) * sc;
                s[h][u] = valid ? acc : -INFINITY;
            }
        }
        // s becomes p = 2^(s - m_new); l and o are rescaled to the new running max.
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            float mx = s[h][0];
#pragma unroll
            for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, s[h][u]);
            const float mn = fmaxf(m[h], mx);
            const float corr = __builtin_amdgcn_exp2f(m[h] - mn);
            m[h] = mn;
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) { s[h][u] = __builtin_amdgcn_exp2f(s[h][u] - mn); ps += s[h][u]; }
            l[h] = fmaf(l[h], corr, ps);
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[h][e] *= corr;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float vf[EPL];
            widen<KV>(vt[u], vf);
#pragma unroll
            for (int h = 0; h < GT; ++h)
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(s[h][u], vf[e], o[h][e]);
        }
    };

    // Software pipeline over two register buffers: while one tile is computed the loads of
    // the next are in flight. The whole byte offset sits in the per-lane offset (the scalar
    // offset is not range-checked), so rows at or past r1 read as zeros.
    Vec ka[kUnroll], va[kUnroll], kb[kUnroll], vb[kUnroll];
    auto load = [&](Vec (&kt)[kUnroll], Vec (&vt)[kUnroll], int tbase) {
        const uint32_t off = lane_off + tbase * ROWB;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            kt[u] = buffer_load<Vec>(krs, off + u * RPL * ROWB, 0);
            vt[u] = buffer_load<Vec>(vrs, off + u * RPL * ROWB, 0);
        }
    };
    int base = r0 + wave * TILE;
    const int ntiles = base < r1 ? (r1 - base + STEP - 1) / STEP : 0;
    if (ntiles > 0) load(ka, va, base);
    // Pairs of tiles with no exit in between, so each prefetch is consumed on every path
    // (a load used on one path only would be sunk to its use by the compiler).
    // The scheduling barriers keep the instruction scheduler from sinking the prefetch
    // loads toward their uses.
    for (int t = 0; t + 1 < ntiles; t += 2) {
        load(kb, vb, base + STEP);
        __builtin_amdgcn_sched_barrier(0);
        process(ka, va, base);
        load(ka, va, base + 2 * STEP);  // past the end this reads zeros and is not processed
        __builtin_amdgcn_sched_barrier(0);
        process(kb, vb, base + STEP);
        base += 2 * STEP;
    }
    if (ntiles & 1) process(ka, va, base);

    // Merge the row groups of this wave (they saw disjoint rows) by their max.
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        float M = m[h];
#pragma unroll
        for (int off = LPR; off < kWave; off *= 2) M = fmaxf(M, __shfl_xor(M, off));
        const float w = __builtin_amdgcn_exp2f(m[h] - M);
        l[h] *= w;
#pragma unroll
        for (int off = LPR; off < kWave; off *= 2) l[h] += __shfl_xor(l[h], off);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float x = o[h][e] * w;
#pragma unroll
            for (int off = LPR; off < kWave; off *= 2) x += __shfl_xor(x, off);
            o[h][e] = x;
        }
        m[h] = M;
    }

    // Merge the waves in LDS and write this split's partial result.
    __shared__ float s_m[kWaves][GT], s_l[kWaves][GT];
    __shared__ float s_o[kWaves][GT][D];
    if (grp == 0) {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) s_o[wave][h][sub * EPL + e] = o[h][e];
            if (sub == 0) { s_m[wave][h] = m[h]; s_l[wave][h] = l[h]; }
        }
    }
    __syncthreads();
    const bool direct = DIRECT && nsplit_b == 1;
    for (int idx = threadIdx.x; idx < GT * D; idx += kBlock) {
        const int h = idx / D, d = idx % D;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
        float Ls = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);
            Ls = fmaf(s_l[w][h], f, Ls);
            O = fmaf(s_o[w][h][d], f, O);
        }
        if (direct) {
            a.out[((size_t)b * h_q + h0 + h) * D + d] = O * vscale / Ls;
        } else {
            const size_t pidx = ((size_t)b * h_q + h0 + h) * a.n_splits + split;
            a.part_o[pidx * D + d] = O * vscale;
            if (d == 0) { a.part_ml[pidx * 2 + 0] = M; a.part_ml[pidx * 2 + 1] = Ls; }
        }
    }
}

// One workgroup per (sequence, query head): merge its splits by log-sum-exp weights.
// skip_single: sequences with one split were already written by the split kernel.
template <int D>
__global__ __launch_bounds__(kCombineBlock) void lse_combine_kernel(
    const int32_t *__restrict__ lens, const float *__restrict__ part_ml,
    const float *__restrict__ part_o, float *__restrict__ out, int32_t *__restrict__ err,
    int h_q, int chunk, int n_splits, int max_len, int skip_single) {
    constexpr int SG = kCombineBlock / D;  // split groups working side by side
    const int bh = blockIdx.x;
    const int b = bh / h_q;
    const int L = lens[b];
    float *dst = out + (size_t)bh * D;
    if (L < 1 || L > max_len) {
        for (int d = threadIdx.x; d < D; d += kCombineBlock) dst[d] = 0.f;
        if (threadIdx.x == 0) atomicOr(err, DA_DEV_ERR_LEN_RANGE);
        return;
    }
    const int ns = (L + chunk - 1) / chunk;
    if (skip_single && ns == 1) return;
    const float *ml = part_ml + (size_t)bh * n_splits * 2;
    const float *po = part_o + (size_t)bh * n_splits * D;

    __shared__ float red[kCombineBlock / kWave];
    __shared__ float s_acc[SG][D], s_l[SG][D];
    float M = kNegBig;
    for (int s = threadIdx.x; s < ns; s += kCombineBlock) M = fmaxf(M, ml[2 * s]);
#pragma unroll
    for (int off = 1; off < kWave; off *= 2) M = fmaxf(M, __shfl_xor(M, off));
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = M;
    __syncthreads();
    M = red[0];
#pragma unroll
    for (int w = 1; w < kCombineBlock / kWave; ++w) M = fmaxf(M, red[w]);

    const int d = threadIdx.x % D, sg = threadIdx.x / D;
    float acc = 0.f, ls = 0.f;
#pragma unroll 4
    for (int s = sg; s < ns; s += SG) {
        const float f = __builtin_amdgcn_exp2f(ml[2 * s] - M);
        ls = fmaf(ml[2 * s + 1], f, ls);
        acc = fmaf(po[(size_t)s * D + d], f, acc);
    }
    s_acc[sg][d] = acc;
    s_l[sg][d] = ls;
    __syncthreads();
    if (sg == 0) {
        float a = s_acc[0][d], z = s_l[0][d];
#pragma unroll
        for (int i = 1; i < SG; ++i) { a += s_acc[i][d]; z += s_l[i][d]; }
        dst[d] = a / z;
    }
}

// ------------------------------------------------------------------ host side
thread_local char g_last_error[512];

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dt) { return dt == DA_F32 ? 4 : dt == DA_BF16 ? 2 : dt == DA_FP8_E4M3FN ? 1 : 0; }

int validate(const da_desc *d) {
    if (!d) return fail(DA_ERR_INVALID_ARG, "desc is NULL");
    if (d->batch < 1 || d->h_q < 1 || d->h_kv < 1 || d->cap < 1 || d->d_k < 1 || d->d_v < 1)
        return fail(DA_ERR_INVALID_ARG, "batch, heads, head sizes and cap must be positive");
    if (d->batch > 65535 || d->h_q > 65535)
        return fail(DA_ERR_UNSUPPORTED, "batch and h_q are limited to 65535 (grid dimensions)");
    if (d->h_q % d->h_kv)
        return fail(DA_ERR_INVALID_ARG, "h_q (%d) is not a multiple of h_kv (%d)", d->h_q, d->h_kv);
    if (!std::isfinite(d->scale)) return fail(DA_ERR_INVALID_ARG, "scale is not finite");
    if (d->chunk_rows < 0 || d->chunk_rows % 256)
        return fail(DA_ERR_INVALID_ARG, "chunk_rows must be 0 or a positive multiple of 256");
    if (!elem_size(d->q_dtype) || !elem_size(d->kv_dtype))
        return fail(DA_ERR_INVALID_ARG, "unknown dtype code");
    if (d->d_k != d->d_v || (d->d_k != 64 && d->d_k != 128))
        return fail(DA_ERR_UNSUPPORTED, "head sizes d_k = d_v in {64, 128} are supported (got %d, %d)",
                    d->d_k, d->d_v);
    const bool ok = (d->q_dtype == DA_F32 && d->kv_dtype == DA_F32) ||
                    (d->q_dtype == DA_BF16 && d->kv_dtype == DA_BF16) ||
                    (d->q_dtype == DA_BF16 && d->kv_dtype == DA_FP8_E4M3FN);
    if (!ok) return fail(DA_ERR_UNSUPPORTED, "dtype pair (q %d, kv %d) is not built", d->q_dtype, d->kv_dtype);
    return DA_OK;
}

// Workspace layout: [error word, padded to 256 B][split (max, sum) pairs,
// B*h_q*n_splits*2 fp32][split output rows, B*h_q*n_splits*d_v fp32], each section starting
// on a 256-byte boundary.
struct Plan {
    int chunk, n_splits, gt;
    size_t ml_off, o_off, bytes;
};

int heads_per_block(int g) { return g % 4 == 0 ? 4 : g % 2 == 0 ? 2 : 1; }

// Rows per split: the largest power-of-two multiple of 256 (up to 4096) that still gives
// at least 2048 workgroups at max_len, so that 256 CUs stay busy, and the longest
// sequence is cut in as few splits as that allows.
int choose_chunk(const da_desc *d, int max_len, int gt) {
    const long blocks_per_split = (long)d->batch * d->h_kv * (d->h_q / d->h_kv / gt);
    int chunk = 256;
    while (chunk < 4096 && blocks_per_split * ((max_len + 2 * chunk - 1) / (2 * chunk)) >= 2048) chunk *= 2;
    return chunk;
}

int make_plan(const da_desc *d, int max_len, Plan *p) {
    int rc = validate(d);
    if (rc) return rc;
    if (max_len < 1 || max_len > d->cap)
        return fail(DA_ERR_INVALID_ARG, "max_len (%d) must be in [1, cap = %d]", max_len, d->cap);
    p->gt = heads_per_block(d->h_q / d->h_kv);
    p->chunk = d->chunk_rows ? d->chunk_rows : choose_chunk(d, max_len, p->gt);
    p->n_splits = (max_len + p->chunk - 1) / p->chunk;

    const size_t rows = (size_t)d->batch * d->h_q * p->n_splits;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    p->ml_off = kHeaderBytes;
    p->o_off = p->ml_off + up(rows * 2 * sizeof(float));
    p->bytes = p->o_off + up(rows * d->d_v * sizeof(float));
    return DA_OK;
}

int launch_status(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return DA_OK;
}

template <int KV, int D, bool DIRECT>
void launch_split_gt(int gt, dim3 grid, hipStream_t st, const SplitArgs &args) {
    switch (gt) {
    case 4: hipLaunchKernelGGL((split_kv_attn_kernel<KV, D, 4, DIRECT>), grid, dim3(kBlock), 0, st, args); break;
    case 2: hipLaunchKernelGGL((split_kv_attn_kernel<KV, D, 2, DIRECT>), grid, dim3(kBlock), 0, st, args); break;
    default: hipLaunchKernelGGL((split_kv_attn_kernel<KV, D, 1, DIRECT>), grid, dim3(kBlock), 0, st, args); break;
    }
}

template <bool DIRECT>
void launch_split(int kv, int d, int gt, dim3 grid, hipStream_t st, const SplitArgs &args) {
    if (kv == DA_F32) {
        if (d == 64) launch_split_gt<DA_F32, 64, DIRECT>(gt, grid, st, args);
        else launch_split_gt<DA_F32, 128, DIRECT>(gt, grid, st, args);
    } else if (kv == DA_BF16) {
        if (d == 64) launch_split_gt<DA_BF16, 64, DIRECT>(gt, grid, st, args);
        else launch_split_gt<DA_BF16, 128, DIRECT>(gt, grid, st, args);
    } else {
        if (d == 64) launch_split_gt<DA_FP8_E4M3FN, 64, DIRECT>(gt, grid, st, args);
        else launch_split_gt<DA_FP8_E4M3FN, 128, DIRECT>(gt, grid, st, args);
    }
}

// Checks the run arguments and launches the split kernel: with out non-NULL, sequences that
// fit one split are written to out directly (decode_attn_run); otherwise every split writes
// its partial result (decode_attn_partial).
int run_split(const da_desc *desc, const void *q, const void *k_cache, const void *v_cache, const int32_t *lens,
              int32_t max_len, const float *kv_scales, float *out, void *workspace, size_t ws_bytes,
              void *stream, const char *who) {
    Plan p;
    int rc = make_plan(desc, max_len, &p);
    if (rc) return rc;
    if (!q || !k_cache || !v_cache || !lens || !workspace)
        return fail(DA_ERR_INVALID_ARG, "%s: a buffer pointer is NULL", who);
    if (desc->kv_dtype == DA_FP8_E4M3FN && !kv_scales)
        return fail(DA_ERR_INVALID_ARG, "%s: an fp8 cache needs kv_scales", who);
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace) ||
        (out && !aligned16(out)))
        return fail(DA_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", who);
    if (ws_bytes < p.bytes)
        return fail(DA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", who, ws_bytes, p.bytes);
    char *ws = static_cast<char *>(workspace);
    SplitArgs args;
    args.q = q;
    args.kc = k_cache;
    args.vc = v_cache;
    args.lens = lens;
    args.kv_scales = kv_scales;
    args.part_ml = reinterpret_cast<float *>(ws + p.ml_off);
    args.part_o = reinterpret_cast<float *>(ws + p.o_off);
    args.out = out;
    args.err = reinterpret_cast<int32_t *>(ws);
    args.h_q = desc->h_q;
    args.h_kv = desc->h_kv;
    args.cap = desc->cap;
    args.chunk = p.chunk;
    args.n_splits = p.n_splits;
    args.max_len = max_len;
    args.qk_scale = desc->scale * kLog2e;
    const int g = desc->h_q / desc->h_kv;
    const dim3 grid(p.n_splits, desc->h_kv * (g / p.gt), desc->batch);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (out)
        launch_split<true>(desc->kv_dtype, desc->d_k, p.gt, grid, st, args);
    else
        launch_split<false>(desc->kv_dtype, desc->d_k, p.gt, grid, st, args);
    return launch_status("split_kv_attn_kernel");
}

int run_combine(const da_desc *desc, const int32_t *lens, int32_t max_len, float *out, void *workspace,
                size_t ws_bytes, void *stream, int skip_single, const char *who) {
    Plan p;
    int rc = make_plan(desc, max_len, &p);
    if (rc) return rc;
    if (!lens || !out || !workspace) return fail(DA_ERR_INVALID_ARG, "%s: a pointer is NULL", who);
    if (!aligned16(out) || !aligned16(workspace))
        return fail(DA_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", who);
    if (ws_bytes < p.bytes)
        return fail(DA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", who, ws_bytes, p.bytes);
    char *ws = static_cast<char *>(workspace);
    const float *ml = reinterpret_cast<const float *>(ws + p.ml_off);
    const float *po = reinterpret_cast<const float *>(ws + p.o_off);
    int32_t *err = reinterpret_cast<int32_t *>(ws);
    const dim3 grid(desc->batch * desc->h_q);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (desc->d_v == 64)
        hipLaunchKernelGGL(lse_combine_kernel<64>, grid, dim3(kCombineBlock), 0, st, lens, ml, po, out, err,
                           desc->h_q, p.chunk, p.n_splits, max_len, skip_single);
    else
        hipLaunchKernelGGL(lse_combine_kernel<128>, grid, dim3(kCombineBlock), 0, st, lens, ml, po, out, err,
                           desc->h_q, p.chunk, p.n_splits, max_len, skip_single);
    return launch_status("lse_combine_kernel");
}

}  // namespace

// ------------------------------------------------------------------ C ABI
extern "C" {

const char *da_status_string(int status) {
    switch (status) {
    case DA_OK: return "ok";
    case DA_ERR_INVALID_ARG: return "invalid argument";
    case DA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DA_ERR_WORKSPACE: return "workspace too small";
    case DA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

const char *da_last_error(void) { return g_last_error; }

int da_workspace_size(const da_desc *desc, int32_t max_len, size_t *bytes) {
    Plan p;
    const int rc = make_plan(desc, max_len, &p);
    if (rc) return rc;
    if (!bytes) return fail(DA_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = p.bytes;
    return DA_OK;
}

int da_plan(const da_desc *desc, int32_t max_len, int32_t *chunk_rows, int32_t *n_splits,
            int32_t *heads_per_block_out) {
    Plan p;
    const int rc = make_plan(desc, max_len, &p);
    if (rc) return rc;
    if (chunk_rows) *chunk_rows = p.chunk;
    if (n_splits) *n_splits = p.n_splits;
    if (heads_per_block_out) *heads_per_block_out = p.gt;
    return DA_OK;
}

int da_workspace_init(void *workspace, size_t ws_bytes, void *stream) {
    if (!workspace || !aligned16(workspace)) return fail(DA_ERR_INVALID_ARG, "workspace is NULL or misaligned");
    if (ws_bytes < kHeaderBytes) return fail(DA_ERR_WORKSPACE, "workspace smaller than its %zu-byte header", kHeaderBytes);
    const size_t words = ws_bytes / 4;
    const unsigned blocks = (unsigned)std::min<size_t>((words + 255) / 256, 2048);
    hipLaunchKernelGGL(workspace_init_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<int32_t *>(workspace), words);
    return launch_status("workspace_init_kernel");
}

int kv_append(const da_desc *desc, void *k_cache, void *v_cache, int32_t *lens, const void *k_new,
              const void *v_new, void *workspace, void *stream) {
    int rc = validate(desc);
    if (rc) return rc;
    if (!k_cache || !v_cache || !lens || !k_new || !v_new)
        return fail(DA_ERR_INVALID_ARG, "kv_append: a buffer pointer is NULL");
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) ||
        (workspace && !aligned16(workspace)))
        return fail(DA_ERR_INVALID_ARG, "kv_append: buffers must be 16-byte aligned");
    const int es = elem_size(desc->kv_dtype);
    const int row_k = desc->d_k * es, row_v = desc->d_v * es;
    hipLaunchKernelGGL(kv_append_kernel, dim3(desc->batch), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<char *>(k_cache), static_cast<char *>(v_cache), lens,
                       static_cast<const char *>(k_new), static_cast<const char *>(v_new),
                       static_cast<int32_t *>(workspace), desc->h_kv, desc->cap, row_k, row_v);
    return launch_status("kv_append_kernel");
}

int decode_attn_partial(const da_desc *desc, const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *lens, int32_t max_len, const float *kv_scales, void *workspace,
                        size_t ws_bytes, void *stream) {
    return run_split(desc, q, k_cache, v_cache, lens, max_len, kv_scales, nullptr, workspace, ws_bytes, stream,
                     "decode_attn_partial");
}

int decode_attn_combine(const da_desc *desc, const int32_t *lens, int32_t max_len, float *out, void *workspace,
                        size_t ws_bytes, void *stream) {
    return run_combine(desc, lens, max_len, out, workspace, ws_bytes, stream, 0, "decode_attn_combine");
}

int decode_attn_run(const da_desc *desc, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *lens, int32_t max_len, const float *kv_scales, float *out, void *workspace,
                    size_t ws_bytes, void *stream) {
    if (!out) return fail(DA_ERR_INVALID_ARG, "decode_attn_run: out is NULL");
    const int rc = run_split(desc, q, k_cache, v_cache, lens, max_len, kv_scales, out, workspace, ws_bytes, stream,
                             "decode_attn_run");
    if (rc) return rc;
    return run_combine(desc, lens, max_len, out, workspace, ws_bytes, stream, 1, "decode_attn_run");
}

int da_read_device_error(const void *workspace, void *stream, int32_t *code) {
    if (!workspace || !code) return fail(DA_ERR_INVALID_ARG, "da_read_device_error: NULL pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t host = 0;
    hipError_t e = hipMemcpyAsync(&host, workspace, sizeof host, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(DA_ERR_LAUNCH, "da_read_device_error: %s", hipGetErrorString(e));
    *code = host;
    return DA_OK;
}

}  // extern "C"
