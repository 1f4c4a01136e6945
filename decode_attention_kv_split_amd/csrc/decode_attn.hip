// gfx950 kernels and C ABI for split-KV decode attention over a growing KV cache.
//
// Method (page "MoA-Structured Decode Attention"): per query head, Step I scores every
// cached K row against q (eq. 1, K read row by row in its stored layout, no transpose),
// Step II takes a max-subtracted softmax of the scores (eq. 2) and Step III sums the V
// rows weighted by it (eq. 3). §5 appends one row per step at its row-major offset, §6
// lets every query head of a group select the group's KV rows instead of a copy.
//
// MI355X mapping (CDNA4, wave64):
//   * Work partition: a unit is (sequence, KV head, head tile of at most 32 of the group's
//     query rows); the rows of all units, concatenated, are cut into equal shares, one per
//     256-thread workgroup, with every workgroup resident (one or two per CU), whatever the
//     length mix. A share cut at unit boundaries gives segments; each segment leaves (max, sum,
//     unnormalised rows) in a partial slot of its own, and the combine kernel merges a unit's
//     segments by their log-sum-exp weights.
//   * Each K and V row is loaded once per head tile and used by all its query rows (the
//     group's g heads at each query position), so KV bytes are read once per group while the
//     group has at most 32 query rows.
//   * Three segment flavours: the vector ALUs (fp32 caches and groups of one or two rows:
//     lanes span the head dimension, coalesced row loads, DPP row sums); the matrix cores with
//     a register ring (bf16: K loaded in A-operand order, V through a per-wave LDS tile read
//     back transposed); the matrix cores with LDS stages filled by DMA (fp8 and int8 codes,
//     widened exactly in registers).
//   * Softmax runs online in fp32 in the base-2 domain (scale * log2 e folded into the score
//     scale, v_exp_f32 for 2^x); the waves of a workgroup merge through LDS at a segment's end.
//   * For latency-bound problems a single-pass kernel does it in one launch: the splits of a
//     unit count their arrivals and the last one merges them.
//   * For a context split over devices, the combine also writes each query row's log-sum-exp
//     (decode_attn_run_lse), and a small kernel merges the parts' results (decode_attn_merge_lse).
//   * No atomics touch the outputs, so results are deterministic run to run.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <type_traits>
#include <map>
#include <mutex>
#include <utility>

#include "decode_attn.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;  // waves per split workgroup
constexpr int kBlock = kWave * kWaves;
constexpr int kUnroll = 4;  // row loads per lane per tile
constexpr int kCombineBlock = 256;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegBig = -3.0e38f;  // finite "minus infinity" for running maxima
// Matrix-core segments rescale their running sums only when a tile's max exceeds the
// exponent reference by this much (base 2), so the exponentials stay below 2^8 = 256.
constexpr float kLazyRescale = 8.f;
constexpr size_t kHeaderBytes = 256;  // error word + padding at the workspace start
constexpr int kCacheLine = 128;        // bytes per vector L1 / L2 cache line

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ element traits
// kEpl elements per lane per row load; the load is kEpl * element-size bytes.
template <int KV> struct Kv;
template <> struct Kv<DA_F32> { static constexpr int kEsz = 4, kEpl = 4; using Vec = uint4; };
template <> struct Kv<DA_BF16> { static constexpr int kEsz = 2, kEpl = 8; using Vec = uint4; };
template <> struct Kv<DA_FP8_E4M3FN> { static constexpr int kEsz = 1, kEpl = 8; using Vec = uint2; };
template <> struct Kv<DA_INT8> { static constexpr int kEsz = 1, kEpl = 8; using Vec = uint2; };

// 8-bit caches hold codes; an element's value is code * its slot's scale.
constexpr bool kv_scaled(int kv) { return kv == DA_FP8_E4M3FN || kv == DA_INT8; }

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

// int8 byte i of w -> fp32 (one v_cvt_f32_i32 with a sign-extended byte operand)
__device__ __forceinline__ float i8_to_f32(uint32_t w, int i) { return (float)(int8_t)(w >> (8 * i)); }

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
    } else if constexpr (KV == DA_INT8) {
        const uint32_t w[2] = {v.x, v.y};
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = i8_to_f32(w[i / 4], i % 4);
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
// raises the split kernel's sustained read rate by 5-10 %. The exception is a load that reads
// half of a 128-byte line whose other half the next load reads (kLoadCached, see the
// matrix-core register ring).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kLoadNonTemporal = 2;
constexpr int kLoadCached = 0;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// The base and size are the same in every lane of the wave; taking them through readfirstlane
// keeps the resource in scalar registers even where the compiler cannot prove that (a
// per-lane resource would wrap every buffer load in a loop over distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    // readfirstlane yields an int: keep each half 32 bits wide (no sign extension)
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// The same resource as four words, for inline assembly.
__device__ __forceinline__ u32x4_t rsrc_words(const void *base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p),
                   (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) & 0xFFFFu,
                   (uint32_t)__builtin_amdgcn_readfirstlane(bytes), (uint32_t)kRsrcWord3};
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)p);
}

// One 1 KiB LDS DMA: lane i's 16 bytes at byte voff of the resource land at LDS byte
// lds + 16 i, non-temporal. It is written as inline assembly because the compiler cannot
// tell which LDS bytes a DMA writes: with the builtin it waits for every DMA in flight
// (vmcnt(0)) before each LDS read, which serialises the stages. The caller orders DMA and
// reads with explicit vmcnt waits and barriers instead. The compiler does not look inside
// the assembly for hazards, so it keeps the wait states itself: five before (a vector
// instruction that wrote one of the resource's scalar registers), one between the write of
// M0 and the DMA that reads it. M0 is a register the compiler reserves, so it warns that the
// clobber may not be honoured (no save or restore around the statement). That is safe here
// only because nothing else in the device code uses M0: in the gfx950 assembly of this file
// every M0 access is one of these statements' own s_mov_b32 (no GPR indexing, s_movrel,
// message or LDS-DMA builtin). Code that adds such a use must not keep M0 live across this.
__device__ __forceinline__ void lds_dma16(u32x4_t rsrc, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}

template <typename Vec, int POLICY = kLoadNonTemporal>
__device__ __forceinline__ Vec buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (sizeof(Vec) == 16) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, POLICY);
        return Vec{x[0], x[1], x[2], x[3]};
    } else {
        const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, POLICY);
        return Vec{x[0], x[1]};
    }
}

// ------------------------------------------------------------------ cross-lane sums
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Exchanges between the four 16-lane rows of a wave by v_permlane16_swap / v_permlane32_swap
// (vector ALU instructions, a few cycles) instead of ds_bpermute (a round trip through the LDS
// unit). With both operands the same value x, the swap of rows leaves lane l holding x of
// lanes l and l ^ 16 (one in each result), and the swap of halves x of lanes l and l ^ 32
// (checked on the device for every lane).
__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over each aligned group of LPR consecutive lanes; every lane gets its group's sum.
// quad_perm [1,0,3,2] and [2,3,0,1] sum a quad; row_half_mirror pairs quads inside
// 8 lanes; row_mirror pairs halves inside a 16-lane row; 32 adds the neighbouring row.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (LPR >= 2) x += dpp<0xB1>(x);
    if constexpr (LPR >= 4) x += dpp<0x4E>(x);
    if constexpr (LPR >= 8) x += dpp<0x141>(x);
    if constexpr (LPR >= 16) x += dpp<0x140>(x);
    if constexpr (LPR >= 32) x = xor16_sum(x);
    return x;
}

// ------------------------------------------------------------------ kernels
// Zeroes n words (the whole workspace: error word and partial results).
__global__ void workspace_init_kernel(int32_t *ws, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        ws[i] = 0;
}

// Plain streaming read for the measured bandwidth ceiling: workgroup w reads its contiguous
// chunk of the buffer with 16-byte non-temporal buffer loads, kStreamUnroll in flight per lane,
// and folds the words into one value per workgroup (so that no load can be dropped).
constexpr int kStreamWorkgroups = 512;
constexpr int kStreamUnroll = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const char *__restrict__ buf, size_t bytes,
                                                          uint32_t chunk, float *__restrict__ sink) {
    const size_t base = (size_t)blockIdx.x * chunk;
    const uint32_t mine = base >= bytes ? 0u : (uint32_t)(bytes - base < chunk ? bytes - base : chunk);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(buf + base, mine);
    uint32_t acc = 0;
    for (uint32_t off = threadIdx.x * 16u; off < mine; off += 256u * 16u * kStreamUnroll) {
        u32x4_t v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + u * 256u * 16u), 0, kLoadNonTemporal);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    __shared__ uint32_t s_acc[kBlock / kWave];
#pragma unroll
    for (int o = 1; o < kWave; o *= 2) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if (threadIdx.x % kWave == 0) s_acc[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = (float)(s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3]);
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

// ------------------------------------------------------------------ work partition
// A "unit" is one (sequence b, KV head kvh, head tile t) with its lens[b] cache rows; a
// sequence whose length is out of range contributes no rows. Units are numbered
// u = (b * h_kv + kvh) * tiles + t and their rows concatenated: unit u starts at row P_u of
// T rows in total. Workgroup w of N takes rows [w*T/N, (w+1)*T/N), so every workgroup gets
// the same number of rows whatever the length mix, and N is chosen so that all of them are
// resident at once. A workgroup's range cut by unit boundaries gives "segments"; the
// (w, u) pairs of all segments form a monotone staircase, so k = w + u numbers them
// uniquely (k < N + units) and indexes their partial results. The workgroups holding a
// unit's first and last rows record themselves for the combine, and every workgroup between
// them leaves a partial for the unit (an empty one when its range holds no rows, which only
// happens with fewer rows than workgroups).
constexpr int kMaxBatch = 1024;
constexpr int kMaxQueries = 1024;  // query rows per sequence in one call

struct Partition {
    int batch, h_kv, tiles, max_len, nwg;
    int append_cap;  // > 0: this pass first appends one row per (sequence, KV head); the cache capacity
    int nq;          // query rows per sequence (> 1: multi-query causal decode)
};

// Rows a pass attends over for a sequence whose stored length is L: with an append in the
// same pass, L + 1 when the new row fits (L in [0, cap)); otherwise L (that append is skipped
// and flagged, as kv_append does).
__device__ __forceinline__ int attended_len(int L, int append_cap) {
    return (append_cap > 0 && L >= 0 && L < append_cap) ? L + 1 : L;
}
// Rows of a sequence of length L in each of its units; 0 (no work, output zeroed and flagged)
// unless 1 <= L <= max_len and L holds the nq query positions.
__device__ __forceinline__ int64_t unit_rows(int L, int max_len, int nq) {
    return (L >= 1 && L >= nq && L <= max_len) ? L : 0;
}
__device__ __forceinline__ int64_t wg_start(int64_t w, int64_t T, int64_t N) { return w * T / N; }

// Exclusive prefix over sequences of their rows in all units, s_pre[0..batch]; s_pre[batch] = T,
// for batches of more than one wave's lanes (smaller ones keep it in registers, in SegWalk).
// The stored lengths land in s_len, so that the walk reads them from LDS, not from memory again.
// Needs batch <= kMaxBatch and blockDim.x == kBlock.
__device__ void sequence_prefix(const int32_t *__restrict__ lens, const Partition &pt, int64_t *s_pre,
                                int64_t *s_wave, int32_t *s_len) {
    const int per = (pt.batch + kBlock - 1) / kBlock;  // <= kMaxBatch / kBlock
    const int64_t upb = (int64_t)pt.h_kv * pt.tiles;
    int64_t local[kMaxBatch / kBlock];
    int64_t sum = 0;
#pragma unroll
    for (int i = 0; i < kMaxBatch / kBlock; ++i) {
        const int bb = threadIdx.x * per + i;
        local[i] = sum;
        if (i < per && bb < pt.batch) {
            const int32_t L = lens[bb];
            s_len[bb] = L;
            sum += unit_rows(attended_len(L, pt.append_cap), pt.max_len, pt.nq) * upb;
        }
    }
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    int64_t incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off *= 2) {
        const int64_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    int64_t wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += s_wave[w];
    const int64_t excl = wbase + incl - sum;
#pragma unroll
    for (int i = 0; i < kMaxBatch / kBlock; ++i) {
        const int bb = threadIdx.x * per + i;
        if (i < per && bb < pt.batch) s_pre[bb] = excl + local[i];
    }
    if (threadIdx.x == kBlock - 1) s_pre[pt.batch] = excl + sum;
    __syncthreads();
}

// Arguments of the split kernel (passed by value as one kernel argument).
struct SplitArgs {
    const void *q, *kc, *vc;
    int32_t *lens;            // written only by the single-pass kernel with an append
    const float *kv_scales;   // [B, h_kv, 2] for fp8 / int8 caches, else unused
    float *part_ml, *part_o;  // per segment: [GT][2] (max, sum) and [GT][D] output rows
    float *out;               // decode_attn_run: output rows of units one workgroup covers
    int h_q, cap;
    Partition pt;
    float qk_scale;           // scale * log2(e)
    // fused append (pt.append_cap > 0): the new rows [B, h_kv, row_bytes] of K and V, the
    // workspace copy of the stored lengths (read by the combine, which then updates lens) and
    // the workspace error word
    const void *k_new, *v_new;
    int32_t *lens_copy, *err;
    int row_bytes;
    int shared_lines;  // cache rows do not sit on whole cache lines of their own
    // for the combine: per unit, the workgroups holding its first and its last row
    int2 *unit_wg;
    int dv;  // output row length (the partial rows' stride)
    // a KV group's g * nq query rows are cut into pt.tiles head tiles of gt rows (the last may
    // hold fewer); gt is also the per-segment stride of the partial arrays
    int gt, grp_rows;
    // single pass: splits per unit, and the arrival counters (per sequence, per unit; at zero
    // between launches)
    int nsplit;
    int32_t *seq_cnt, *unit_cnt;
};

// The query rows of a (sequence b, KV head kvh) are its g heads at each of the nq query
// positions, g * nq rows taken position-major (row r: position r / g, head kvh * g + r % g);
// a head tile holds rows h0 - kvh * g .. of them. For head slot hh of the tile: `row` indexes
// the [d] vectors of q and out ([B, nq, h_q, d]), t is the query's position among the nq,
// and the query attends over rows [0, slen - nq + 1 + t) of a sequence of slen rows (causal:
// its own row and every earlier one). With nq = 1 that is head h0 + hh over all slen rows.
struct QRow {
    size_t row;
    int lim;
};
__device__ __forceinline__ QRow query_row(const SplitArgs &a, int b, int kvh, int h0, int hh, int slen) {
    const int g = a.h_q / a.pt.h_kv;
    const int fr = h0 - kvh * g + hh;
    const int t = fr / g;
    return {((size_t)b * a.pt.nq + t) * a.h_q + kvh * g + fr % g, slen - a.pt.nq + 1 + t};
}

// Steps I-III over rows [r0, r1) of one (sequence b, KV head kvh) for the hv <= GT query rows
// h0 .. h0+hv-1 of a head tile, by the whole workgroup (slots hv .. GT-1 compute on a copy of
// the first row and are never stored). The result (max, sum of exponentials, unnormalised
// output; base-2 domain, V scale applied) goes to segment slot k of the partial arrays, or
// normalised straight to out when `direct` (the segment is the whole unit).
// NW waves per workgroup, U row loads per lane per tile. COH: the partial results are stored
// at agent scope (write-through to the device's coherence point), for a merge by another
// workgroup of the same launch.
template <int KV, int D, int GT, int NW = kWaves, int U = kUnroll, bool COH = false>
__device__ __forceinline__ void attend_segment(const SplitArgs &a, int b, int kvh, int h0, int hv, int r0, int r1,
                                               size_t k, bool direct, int slen) {
    using T = Kv<KV>;
    using Vec = typename T::Vec;
    constexpr int EPL = T::kEpl;
    constexpr int LPR = D / EPL;         // lanes per row
    constexpr int RPL = kWave / LPR;     // rows per wave load
    constexpr int TILE = U * RPL;        // rows per wave per iteration
    constexpr int STEP = TILE * NW;      // rows per workgroup per iteration
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int grp = lane / LPR, sub = lane % LPR;

    const size_t slot = (size_t)b * a.pt.h_kv + kvh;
    constexpr uint32_t ROWB = D * T::kEsz;  // bytes per cache row
    // Resources cover rows [0, r1) of this (sequence, KV head): loads of rows past the
    // segment's end return zeros (and are masked out of the softmax below).
    const size_t slot_bytes = (size_t)a.cap * ROWB;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const char *>(a.kc) + slot * slot_bytes, r1 * ROWB);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(static_cast<const char *>(a.vc) + slot * slot_bytes, r1 * ROWB);
    const uint32_t lane_off = grp * ROWB + sub * (uint32_t)sizeof(Vec);
    float vscale = 1.f, sc = a.qk_scale;
    if constexpr (kv_scaled(KV)) {
        sc *= a.kv_scales[slot * 2 + 0];
        vscale = a.kv_scales[slot * 2 + 1];
    }

    // This lane's slice of q for the GT heads: fp32 values, or packed bf16 pairs for the
    // bf16 dot instruction; each head's end of rows (the segment's, or the causal bound).
    float qf[GT][EPL];
    uint32_t qp[GT][EPL / 2];
    int rend[GT];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        const QRow qr = query_row(a, b, kvh, h0, h < hv ? h : 0, slen);
        rend[h] = min(r1, qr.lim);
        const size_t qoff = qr.row * D + sub * EPL;
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
    auto process = [&](const Vec (&kt)[U], const Vec (&vt)[U], int tbase) {
        float s[GT][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = tbase + u * RPL + grp;
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
                s[h][u] = row < rend[h] ? acc : -INFINITY;
            }
        }
        // s becomes p = 2^(s - m_new); l and o are rescaled to the new running max.
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            float mx = s[h][0];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[h][u]);
            const float mn = fmaxf(m[h], mx);
            const float corr = __builtin_amdgcn_exp2f(m[h] - mn);
            m[h] = mn;
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) { s[h][u] = __builtin_amdgcn_exp2f(s[h][u] - mn); ps += s[h][u]; }
            l[h] = fmaf(l[h], corr, ps);
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[h][e] *= corr;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
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
    Vec ka[U], va[U], kb[U], vb[U];
    auto load = [&](Vec (&kt)[U], Vec (&vt)[U], int tbase) {
        const uint32_t off = lane_off + tbase * ROWB;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            kt[u] = buffer_load<Vec>(krs, off + u * RPL * ROWB, 0);
            vt[u] = buffer_load<Vec>(vrs, off + u * RPL * ROWB, 0);
        }
    };
    int base = r0 + wave * TILE;
    const int ntiles = base < r1 ? (r1 - base + STEP - 1) / STEP : 0;
    if (ntiles > 0) load(ka, va, base);
    // Pairs of tiles with no exit in between, so each prefetch is consumed on every path
    // (a load used on one path only would be sunk to its use by the compiler); the
    // scheduling barriers keep the instruction scheduler from sinking the prefetch loads.
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

    // Merge the waves in LDS and write this segment's result.
    __shared__ float s_m[NW][GT], s_l[NW][GT];
    __shared__ float s_o[NW][GT][D];
    if (grp == 0) {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) s_o[wave][h][sub * EPL + e] = o[h][e];
            if (sub == 0) { s_m[wave][h] = m[h]; s_l[wave][h] = l[h]; }
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < hv * D; idx += NW * kWave) {
        const int h = idx / D, d = idx % D;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
        float Ls = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);
            Ls = fmaf(s_l[w][h], f, Ls);
            O = fmaf(s_o[w][h][d], f, O);
        }
        if (direct) {
            a.out[query_row(a, b, kvh, h0, h, slen).row * D + d] = O * vscale / Ls;
        } else {
            if constexpr (COH) {
                __hip_atomic_store(&a.part_o[(k * a.gt + h) * D + d], O * vscale, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                if (d == 0) {
                    __hip_atomic_store(&a.part_ml[(k * a.gt + h) * 2 + 0], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(&a.part_ml[(k * a.gt + h) * 2 + 1], Ls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            } else {
                a.part_o[(k * a.gt + h) * D + d] = O * vscale;
                if (d == 0) { a.part_ml[(k * a.gt + h) * 2 + 0] = M; a.part_ml[(k * a.gt + h) * 2 + 1] = Ls; }
            }
        }
    }
    __syncthreads();  // the LDS arrays are reused by the next segment
}

// ------------------------------------------------------------------ MFMA flavour (groups of 3 or more query rows)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

typedef int i32x2_t __attribute__((ext_vector_type(2)));

// s_waitcnt immediate (gfx9 layout) that waits until at most n vector-memory operations of
// this wave are outstanding, without waiting on the LDS / export counters.
constexpr int vmcnt_only(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Two e4m3fn codes (bytes 2*HI, 2*HI+1 of w) -> two bf16 packed in a word, in one
// v_cvt_scalef32_pk_bf16_fp8 with scale 1; exact, since every e4m3fn value is a bf16 value
// (checked on the device for all 256 codes and both halves). The result is read as one
// 32-bit word: extracting its second element as a separate bf16 is mis-compiled (the low
// half is stored twice).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Eight e4m3fn codes as bf16x8, exactly.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(const uint2 &v) {
    return uint4{fp8x2_to_bf16x2<false>(v.x), fp8x2_to_bf16x2<true>(v.x), fp8x2_to_bf16x2<false>(v.y),
                 fp8x2_to_bf16x2<true>(v.y)};
}

// Steps I-III on the matrix cores for query heads h0 .. h0+GT-1 of one (sequence, KV head).
// Per 16-row tile and wave:
//   * Step I as S = K_tile . Q^T with v_mfma_f32_16x16x32_bf16: the K rows are the A operand
//     as stored (lane l holds row l%16, elements 8*(l/16) .. of each 32-wide block), q of 16
//     heads is the B operand. The result gives lane l the scores of rows 4*(l/16)+i (i < 4)
//     for head l%16.
//   * Step II online on that layout: the tile max per head reduces over the 4 lane groups;
//     O is rescaled only when some head's max grew.
//   * Step III transposed, O^T += V_tile^T . P^T with v_mfma_f32_16x16x16_bf16: V, staged in
//     LDS as bf16 and read back with ds_read_b64_tr_b16 (lane l: d column l%16, rows
//     4*(l/16) ..), is the A operand, and the score layout above is exactly the B-operand
//     layout of P^T. Lane l then holds d = 4*(l/16)+i of head l%16: the head's rescale factor
//     is its own, with no exchange between lanes. P is split into bf16 hi + lo parts (two
//     MFMAs) so that P.V keeps ~16 bits of P's precision.
// GW = 16 or 32 query-row slots (HT = 1 or 2 MFMA tiles of 16); slots past the tile's hv rows
// hold zero queries and are never stored.
template <int D, int GW>
struct MfmaAttn {
    static constexpr int HT = GW / 16;
    static constexpr int KB = D / 32;  // 32-wide k blocks of Step I
    static constexpr int NB = D / 16;  // 16-wide d blocks of Step III
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

    bf16x8_t qb[HT][KB];
    float m[HT], lp[HT];
    f32x4_t o[HT][NB];
    float sc;
    int lane, lr, lg, wave;
    int lim[HT];  // end of the rows this lane's head (ht*16 + l%16) may see (causal bound)

    // q^T as the B operand of Step I: lane l holds q[head ht*16 + l%16][kb*32 + 8*(l/16) ..+8].
    __device__ __forceinline__ void init(const SplitArgs &a, int b, int kvh, int h0, int hv, int slen,
                                         float score_scale) {
        lane = threadIdx.x % kWave;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        lr = lane % 16;
        lg = lane / 16;
        sc = score_scale;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int head = ht * 16 + lr;
            const QRow qr = query_row(a, b, kvh, h0, head < hv ? head : 0, slen);
            lim[ht] = qr.lim;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                uint4 x = {0u, 0u, 0u, 0u};
                if (head < hv)
                    x = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + qr.row * D + kb * 32 +
                                                          8 * lg);
                qb[ht][kb] = __builtin_bit_cast(bf16x8_t, x);
            }
            m[ht] = kNegBig;
            lp[ht] = 0.f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) o[ht][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }

    // One tile of rows tb .. tb+15 (rows at or past r1, or past a head's causal bound, masked):
    // ka = the K rows as A operands;
    // vaddr(nb) = this lane's LDS address for the transpose read of d block nb.
    template <class VAddr>
    __device__ __forceinline__ void tile(const bf16x8_t (&ka)[KB], VAddr &&vaddr, int tb, int r1) {
        bool grew = false;
        float x[HT][4], tmax[HT];
        bf16x4_t phi[HT], plo[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb], qb[ht][kb], sacc, 0, 0, 0);
            const int rend = min(r1, lim[ht]);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[ht][i] = (tb + 4 * lg + i < rend) ? sacc[i] * sc : -INFINITY;
            tmax[ht] = xor32_max(xor16_max(fmaxf(fmaxf(x[ht][0], x[ht][1]), fmaxf(x[ht][2], x[ht][3]))));
            grew |= tmax[ht] > m[ht] + kLazyRescale;
        }
        // Lazy rescaling: m is the reference the exponentials are taken against, not the exact
        // running max; it moves (and O and the sums are rescaled) only when some head's tile
        // max passes it by kLazyRescale, so p = 2^(s - m) stays below 2^kLazyRescale.
        const bool rescale = __builtin_amdgcn_ballot_w64(grew);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            float corr = 1.f;
            if (rescale) {
                const float mn = fmaxf(m[ht], tmax[ht]);
                corr = __builtin_amdgcn_exp2f(m[ht] - mn);
                m[ht] = mn;
            }
            float p[4], ps = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) { p[i] = __builtin_amdgcn_exp2f(x[ht][i] - m[ht]); ps += p[i]; }
            lp[ht] = fmaf(lp[ht], corr, ps);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                phi[ht][i] = (__bf16)p[i];
                plo[ht][i] = (__bf16)(p[i] - (float)phi[ht][i]);
            }
            if (rescale) {
                // O is held transposed (d rows 4*(l/16)+i of head l%16): the factor is in-lane
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    o[ht][nb][0] *= corr; o[ht][nb][1] *= corr; o[ht][nb][2] *= corr; o[ht][nb][3] *= corr;
                }
            }
        }
        // O^T += V_tile^T . P^T: the transposed V read (lane l: column l%16 of d block nb, rows
        // 4*(l/16) ..) is the A operand of V^T, the score layout the B operand of P^T
        // all hi products first, then all lo ones: the two MFMAs into one accumulator are NB
        // (or NB * HT) instructions apart instead of back to back
        bf16x4_t bvs[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            bvs[nb] = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)vaddr(nb)));
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                o[ht][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bvs[nb], phi[ht], o[ht][nb], 0, 0, 0);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                o[ht][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bvs[nb], plo[ht], o[ht][nb], 0, 0, 0);
    }

    // Merge of the four waves: each puts its (max, sum) and O into its own LDS slot; after one
    // barrier every thread merges float4 columns of the tile's rows over the four slots by
    // their log-sum-exp weights (Step II's normalisation over the union of the waves' rows) and
    // writes them, so the outputs leave from all four waves at once. s_oo holds kWaves * HT*16
    // rows of kRowO floats (one head's D outputs and a 16-byte pad, so that the 16 heads of a
    // wave's store land on distinct banks), s_mm / s_ll kWaves * HT*16 each. (The first
    // version merged pairwise, (0,2), (1,3) then (0,1): four barriers, and wave 0 wrote every
    // output.)
    static constexpr int kRowO = D + 4;
    __device__ __forceinline__ void finish(const SplitArgs &a, int b, int kvh, int h0, int hv, int slen, size_t k,
                                           bool direct, float vscale, float *s_oo, float *s_mm, float *s_ll) {
        constexpr int HP = HT * 16;
        constexpr int C4 = D / 4;  // float4 columns of a row
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {  // the lane groups share each head's max: sums add
            lp[ht] = xor32_sum(xor16_sum(lp[ht]));
        }
        __syncthreads();  // every wave is done with the LDS the merge reuses
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            if (lg == 0) {
                s_mm[wave * HP + ht * 16 + lr] = m[ht];
                s_ll[wave * HP + ht * 16 + lr] = lp[ht];
            }
            // O^T layout: lane l holds d = nb*16 + 4*(l/16) + i of head ht*16 + l%16
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                *reinterpret_cast<f32x4_t *>(&s_oo[(wave * HP + ht * 16 + lr) * kRowO + nb * 16 + 4 * lg]) = o[ht][nb];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < hv * C4; i += kBlock) {
            const int head = i / C4, c4 = i % C4;
            float M = s_mm[head];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_mm[w * HP + head]);
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float f = __builtin_amdgcn_exp2f(s_mm[w * HP + head] - M);
                L = fmaf(s_ll[w * HP + head], f, L);
                const f32x4_t x = *reinterpret_cast<const f32x4_t *>(&s_oo[(w * HP + head) * kRowO + 4 * c4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(x[e], f, acc[e]);
            }
            const f32x4_t v = acc * vscale;
            if (direct) {
                const size_t row = query_row(a, b, kvh, h0, head, slen).row;
                *reinterpret_cast<f32x4_t *>(&a.out[row * D + 4 * c4]) = v / L;
            } else {
                *reinterpret_cast<f32x4_t *>(&a.part_o[(k * a.gt + head) * D + 4 * c4]) = v;
                if (c4 == 0) {
                    a.part_ml[(k * a.gt + head) * 2 + 0] = M;
                    a.part_ml[(k * a.gt + head) * 2 + 1] = L;
                }
            }
        }
        __syncthreads();  // the LDS arrays are reused by the next segment
    }
};

// Matrix-core segment with the tiles staged through registers (bf16 caches): K rows are loaded
// straight into A-operand order and V rows are stored row-major in the wave's LDS tile for the
// transpose read.
template <int KV, int D, int GW, int NBUF>
__device__ __forceinline__ void attend_segment_mfma(const SplitArgs &a, int b, int kvh, int h0, int hv, int r0,
                                                    int r1, size_t k, bool direct, int slen) {
    static_assert(KV == DA_BF16, "the register-ring segment takes bf16 caches");
    using LVec = uint4;  // 8 elements
    using A = MfmaAttn<D, GW>;
    constexpr int KB = A::KB, HP = A::HT * 16;
    constexpr int ESZ = Kv<KV>::kEsz;
    constexpr uint32_t ROWB = D * ESZ;   // bytes per cache row
    constexpr int TR = 16;               // rows per wave tile
    constexpr int STEP = TR * kWaves;    // rows per workgroup step
    constexpr int VROW = D + 8;          // staged V row, bf16 elements (16-byte pad)
    constexpr int VL = D / 8;            // lanes per row of a V load
    constexpr int VRPI = kWave / VL;     // V rows per load instruction
    constexpr int VLD = TR / VRPI;       // V loads per tile

    // Rows of the segment per wave: the whole 64-row steps interleaved by 16-row tile (wave w
    // takes tile w of each step, so a workgroup reads one contiguous 16 KiB run at a time),
    // then the tail of fewer than 64 rows split in four nearly equal parts, one short tile
    // per wave. The waves then reach the merge together; a tail handed out by whole tiles
    // would leave up to one tile more on some waves.
    const int wq = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nfull = (r1 - r0) / STEP, tail = (r1 - r0) % STEP;
    const int ts = r0 + nfull * STEP + tail * wq / kWaves;        // this wave's tail rows
    const int te = r0 + nfull * STEP + tail * (wq + 1) / kWaves;  // [ts, te)
    const size_t slot = (size_t)b * a.pt.h_kv + kvh;
    const size_t slot_bytes = (size_t)a.cap * ROWB;
    // resources of the whole steps (rows below r1) and of this wave's tail (rows below te):
    // rows past them read as zeros without a memory access
    const char *kslot = static_cast<const char *>(a.kc) + slot * slot_bytes;
    const char *vslot = static_cast<const char *>(a.vc) + slot * slot_bytes;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kslot, r1 * ROWB), vrs = make_rsrc(vslot, r1 * ROWB);
    const __amdgpu_buffer_rsrc_t krt = make_rsrc(kslot, te * ROWB), vrt = make_rsrc(vslot, te * ROWB);
    // tile t of this wave: its first row and the end of its rows; tiles past the last start
    // at r1 (nothing fetched, everything masked)
    const int ntiles = nfull + (te > ts ? 1 : 0);
    auto tile_row = [&](int t) { return t < nfull ? r0 + t * STEP + wq * TR : t < ntiles ? ts : r1; };
    auto tile_end = [&](int t) { return t < nfull ? r1 : te; };
    const float vscale = 1.f, sc = a.qk_scale;
    A at;
    at.init(a, b, kvh, h0, hv, slen, sc);
    const int lane = at.lane, wave = at.wave, lr = at.lr, lg = at.lg;
    const int vrow = lane / VL, vcol = (lane % VL) * 8;

    // the waves' V tiles while streaming, the merge's O slots at the end (finish starts and ends
    // with a barrier): one array
    constexpr int kVBytes = kWaves * TR * VROW * 2, kOBytes = kWaves * HP * A::kRowO * 4;
    __shared__ __align__(16) char s_buf[kVBytes > kOBytes ? kVBytes : kOBytes];
    __shared__ float s_mm[kWaves * HP], s_ll[kWaves * HP];
    uint16_t *const s_vw = reinterpret_cast<uint16_t *>(s_buf) + wave * TR * VROW;  // this wave's V tile
    float *const s_oo = reinterpret_cast<float *>(s_buf);

    auto process = [&](const LVec (&kt)[KB], const LVec (&vt)[VLD], int t) {
#pragma unroll
        for (int u = 0; u < VLD; ++u)
            *reinterpret_cast<uint4 *>(&s_vw[(vrow + u * VRPI) * VROW + vcol]) = vt[u];
        bf16x8_t ka[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) ka[kb] = __builtin_bit_cast(bf16x8_t, kt[kb]);
        at.tile(ka, [&](int nb) {
            return (__attribute__((address_space(3))) uint16_t *)s_vw +
                   (4 * lg + lr / 4) * VROW + nb * 16 + 4 * (lane % 4);
        }, tile_row(t), tile_end(t));
    };
    // Software pipeline over a ring of NBUF register buffers: NBUF - 1 tiles of this wave are
    // in flight while one is computed. The ring is unrolled so every buffer index is static;
    // tiles past the segment's end read zeros and are fully masked (p = 0), so every load is
    // consumed on every path (a load used on one path only would be sunk to its use).
    LVec kr[NBUF][KB], vr[NBUF][VLD];
    auto load = [&](LVec (&kt)[KB], LVec (&vt)[VLD], int t) {
        const int tb = tile_row(t);
        const bool in_tail = t >= nfull;
        const __amdgpu_buffer_rsrc_t kr_ = in_tail ? krt : krs, vr_ = in_tail ? vrt : vrs;
        const uint32_t koff = (tb + lr) * ROWB + lg * 8 * ESZ;
        // K in A-operand order reads 64 bytes of each of 16 rows per instruction: the two halves
        // of a 128-byte line come from consecutive loads (k blocks 2i, 2i+1). Cached, the vector
        // L1 serves the second half; with the non-temporal hint it goes to the L2 as a request
        // of its own, and with two workgroups per CU (16 slots) about 2 % of those missed there
        // and fetched the line again (FETCH_SIZE 1.0145 x the algorithmic bytes on the ragged
        // GQA step, against 1.0004 cached, which also runs 1.6 % faster). With 32 slots (one
        // workgroup per CU) the second halves hit the L2 (1.0018) and the hint is kept. V loads
        // read whole rows and keep it too.
        constexpr int kKPolicy = GW == 16 ? kLoadCached : kLoadNonTemporal;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kt[kb] = buffer_load<LVec, kKPolicy>(kr_, koff + kb * 32 * ESZ, 0);
        const uint32_t voff = (tb + vrow) * ROWB + vcol * ESZ;
#pragma unroll
        for (int u = 0; u < VLD; ++u) vt[u] = buffer_load<LVec>(vr_, voff + u * VRPI * ROWB, 0);
    };
    if (ntiles > 0) {
#pragma unroll
        for (int j = 0; j + 1 < NBUF; ++j) load(kr[j], vr[j], j);
        for (int t = 0; t < ntiles; t += NBUF) {
#pragma unroll
            for (int j = 0; j < NBUF; ++j) {
                load(kr[(j + NBUF - 1) % NBUF], vr[(j + NBUF - 1) % NBUF], t + j + NBUF - 1);
                __builtin_amdgcn_sched_barrier(0);
                process(kr[j], vr[j], t + j);
            }
        }
    }
    at.finish(a, b, kvh, h0, hv, slen, k, direct, vscale, s_oo, s_mm, s_ll);
}

// int8 codes on the matrix cores go through fp16, whose 11-bit significand holds 1024 + u
// exactly for any byte u: with the code's sign bit flipped (u = code + 128) and 0x64 as the
// high byte, a half is 1024 + u = code + 1152, two halves per v_perm; a packed subtraction
// of 1152 leaves the code. That costs 1.25 instructions per code, against 1.5 for an exact
// int8 -> bf16 conversion.
// Eight codes -> fp16 code + 1152 (as raw halves).
__device__ __forceinline__ uint4 i8x8_to_f16x8_offset(const uint2 &v) {
    const uint32_t x = v.x ^ 0x80808080u, y = v.y ^ 0x80808080u;
    return uint4{__builtin_amdgcn_perm(0x64646464u, x, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u),
                 __builtin_amdgcn_perm(0x64646464u, y, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, y, 0x04030402u)};
}
// Eight codes -> fp16, exactly (the offset taken off by a packed half subtraction).
__device__ __forceinline__ uint4 i8x8_to_f16x8(const uint2 &v) {
    const uint4 h = i8x8_to_f16x8_offset(v);
    const f16x2_t off = {(_Float16)1152.f, (_Float16)1152.f};
    return uint4{__builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, h.x) - off),
                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, h.y) - off),
                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, h.z) - off),
                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, h.w) - off)};
}

// Matrix-core segment for 8-bit codes (fp8, int8) with workgroup-wide LDS stages filled by DMA
// (buffer_load ... lds), so that no registers hold K or V in flight and 64 KiB per CU are
// outstanding.
//   * A stage holds RS rows of K and V (16 KiB each: 128 rows of d = 128).
//     One DMA instruction fills 1 KiB in lane order. Two layouts:
//       - 128-byte rows (8-bit codes, d = 128): "pieces" of 8 whole rows, so that every DMA
//         instruction reads 8 whole 128-byte lines (half-line reads spread over 16 rows
//         stream 14 % slower, measured). Chunk c of row r of piece m sits at byte
//         m*1024 + ((c ^ key(m))*8 + r)*16, with the swizzle key of piece_key: the K
//         operand reads (16 rows of one chunk) and the V transpose reads (8 rows of pieces
//         m and m+2) then fall on distinct banks.
//       - otherwise every 16-row tile chunk-major: 16-byte chunk c of row r at byte
//         (c*16 + r)*16 (lane i of DMA q: chunk 4q + i/16, row i%16; for 64-byte rows that
//         is 16 whole rows), so the K A operand of k block kb is one contiguous KiB and the
//         V transpose reads of a d block a contiguous 512 bytes.
//     Two stages alternate (separate arrays); all 256 threads fill each; explicit vmcnt waits
//     and barriers mark a stage filled / consumed.
//   * Each wave owns one 16-head tile (its own q operand, running max, sums and O) and a
//     share of the stage's 32-row P.V blocks (Step III by v_mfma_f32_16x16x32_bf16 with P's 8
//     rows per lane taken from the block's two score tiles, V read as codes by
//     ds_read_b64_tr_b8 and widened in registers: fp8 exactly to bf16, int8 to fp16 as
//     code + 1152). Step I uses v_mfma_f32_16x16x32_bf16 (fp8 K widened to bf16 after its LDS
//     read; int8 K exactly to fp16 and the _f16 instruction). Step III is computed
//     transposed, O^T += V^T . P^T (the V read is the A operand, the score layout the B
//     operand), so that each lane holds d rows of its own head and rescales them by that
//     head's factor with no exchange.
//   * At the end the waves holding the same head tile merge through LDS.
// Swizzle key of the piece (8 rows of 128 bytes) at index m of a stage: flips the parity of
// every chunk index in pieces whose Gray code is odd, so that pieces 2t / 2t+1 (one K tile)
// and m / m+2 (the rows one V transpose read gathers) use opposite halves of the banks.
__device__ __forceinline__ int piece_key(int m) { return (m ^ (m >> 1)) & 1; }

template <int KV, int D, int GW>
__device__ __forceinline__ void attend_segment_staged(const SplitArgs &a, int b, int kvh, int h0, int hv, int r0,
                                                      int r1, size_t k, bool direct, int slen) {
    static_assert(Kv<KV>::kEsz == 1, "the LDS-staged segment takes 8-bit codes");
    constexpr int HT = GW / 16;
    constexpr int KB = D / 32, NB = D / 16;
    constexpr int ESZ = Kv<KV>::kEsz;
    constexpr uint32_t ROWB = D * ESZ;         // bytes per cache row
    constexpr int TILE = 16 * ROWB;            // K (or V) bytes of a 16-row tile
    constexpr int HALF = 16384;                // K (or V) bytes per stage
    constexpr int RS = HALF / ROWB;            // rows per stage
    constexpr int PVR = 32;                    // rows per P.V block
    constexpr int NBLK = RS / PVR;             // P.V blocks per stage
    constexpr int WPH = kWaves / HT;           // waves per head tile
    constexpr int IPW = NBLK / WPH;            // blocks per wave per stage
    constexpr int DPW = HALF / 1024 / kWaves;  // K (and V) DMA instructions per wave per stage
    constexpr int VM_STAGE = 2 * DPW;          // DMA ops of one stage per wave
    constexpr bool kLines = ROWB == 128;       // 8-bit codes, d = 128: whole-line DMA layout
    static_assert(NBLK % WPH == 0 && (HALF / 1024) % kWaves == 0, "stage split");
    // int8 goes through fp16: K and V exactly, q scaled by a power of two per head into
    // fp16's range (the factor moves to the score scale), P split into fp16 hi + lo.
    constexpr bool kF16 = KV == DA_INT8;
    // fp16 P is taken 2^7 times larger (at most 2^15 with the lazy rescaling), which keeps
    // small weights out of fp16's subnormals; the segment's sums and rows carry the factor,
    // and its partial reports a maximum 7 lower, which the combine's weights undo
    constexpr float kPShift = kF16 ? 7.f : 0.f;
    using PV = std::conditional_t<kF16, f16x8_t, bf16x8_t>;
    using PE = std::conditional_t<kF16, _Float16, __bf16>;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int lr = lane % 16, lg = lane / 16;
    const int ht = wave % HT;  // this wave's head tile
    const int wb = wave / HT;  // this wave's first P.V block in a stage

    __shared__ __align__(16) char s_a[2 * HALF];
    __shared__ __align__(16) char s_b[2 * HALF];
    __shared__ float s_mm[kWaves][16], s_ll[kWaves][16];
    typedef __attribute__((address_space(3))) char lds_char;

    const size_t slot = (size_t)b * a.pt.h_kv + kvh;
    const size_t slot_bytes = (size_t)a.cap * ROWB;
    const u32x4_t krs = rsrc_words(static_cast<const char *>(a.kc) + slot * slot_bytes, r1 * ROWB);
    const u32x4_t vrs = rsrc_words(static_cast<const char *>(a.vc) + slot * slot_bytes, r1 * ROWB);
    float vscale = 1.f, sc = a.qk_scale;
    if constexpr (kv_scaled(KV)) {
        sc *= a.kv_scales[slot * 2 + 0];
        vscale = a.kv_scales[slot * 2 + 1];
    }
    // q^T of this wave's 16 heads as the B operand of Step I (zero past GT), and the end of
    // the rows this lane's head may see (the segment's, or the causal bound)
    uint4 qb[KB];  // bf16, or fp16 for int8
    int rend;
    float scl = sc;  // this lane's head's score scale
    {
        const int head = ht * 16 + lr;
        const QRow qr = query_row(a, b, kvh, h0, head < hv ? head : 0, slen);
        rend = min(r1, qr.lim);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            uint4 x = {0u, 0u, 0u, 0u};
            if (head < hv)
                x = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + qr.row * D + kb * 32 + 8 * lg);
            qb[kb] = x;
        }
        if constexpr (kF16) {
            // the head's largest |q| (its elements sit in lanes l, l^16, l^32, l^48), then
            // q * 2^-e in fp16 with the largest at 2^14 .. 2^15, in fp16's normal range (exact:
            // a bf16 significand fits fp16's; e stays >= -100 so that 2^-e is a finite float)
            float mx = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const uint32_t w4[4] = {qb[kb].x, qb[kb].y, qb[kb].z, qb[kb].w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(w4[j] << 16)), fabsf(__uint_as_float(w4[j] & 0xffff0000u))));
            }
            mx = xor32_max(xor16_max(mx));
            int ex = 0;
            (void)frexpf(mx, &ex);  // mx < 2^ex
            const int e = max(-100, ex - 15);
            const float down = ldexpf(1.f, -e);
            scl = ldexpf(sc, e);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const uint32_t w4[4] = {qb[kb].x, qb[kb].y, qb[kb].z, qb[kb].w};
                uint32_t h4[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f16x2_t hv = {(_Float16)(__uint_as_float(w4[j] << 16) * down),
                                        (_Float16)(__uint_as_float(w4[j] & 0xffff0000u) * down)};
                    h4[j] = __builtin_bit_cast(uint32_t, hv);
                }
                qb[kb] = uint4{h4[0], h4[1], h4[2], h4[3]};
            }
        }
    }
    float m = kNegBig, lp = 0.f;
    f32x4_t o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Rows at or past r1 are never fetched, so their stage bytes must be finite: the stages
    // start zeroed (they may hold the previous segment's merge data otherwise).
    for (int i = threadIdx.x; i < 2 * HALF / 16; i += kBlock) {
        reinterpret_cast<uint4 *>(s_a)[i] = uint4{0u, 0u, 0u, 0u};
        reinterpret_cast<uint4 *>(s_b)[i] = uint4{0u, 0u, 0u, 0u};
    }
    __syncthreads();

    const uint32_t lds_a = lds_addr(s_a), lds_b = lds_addr(s_b);
    auto issue = [&](uint32_t st, int sb) {
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
            const int x = wave * DPW + j;  // the stage's x-th KiB
            uint32_t off;
            if constexpr (kLines) {  // piece x: rows 8x .. 8x+7, lane i -> row i % 8, chunk (i / 8) ^ key
                off = (sb + 8 * x + lane % 8) * ROWB + (((lane / 8) ^ piece_key(x)) * 16);
            } else {  // tile x / (TILE/1024), part x % (TILE/1024)
                const int t = x / (TILE / 1024), qq = x % (TILE / 1024);
                off = (sb + 16 * t + lr) * ROWB + (4 * qq + lg) * 16;
            }
            lds_dma16(krs, off, st + x * 1024);
            lds_dma16(vrs, off, st + HALF + x * 1024);
        }
    };

    // Online softmax over NR rows held 4 per 16-row score tile: x[] are the scaled, masked
    // scores; returns P split into bf16 hi / lo in the lane's row order and rescales O.
    // (lazy rescaling as in MfmaAttn::tile: m moves only when a tile max passes it by
    // kLazyRescale)
    auto softmax = [&](float *x, PV &phi, PV &plo, int nr) {
        float tmax = x[0];
        for (int i = 1; i < nr; ++i) tmax = fmaxf(tmax, x[i]);
        tmax = xor32_max(xor16_max(tmax));
        float corr = 1.f;
        const bool rescale = __builtin_amdgcn_ballot_w64(tmax > m + kLazyRescale);
        if (rescale) {
            const float mn = fmaxf(m, tmax);
            corr = __builtin_amdgcn_exp2f(m - mn);
            m = mn;
        }
        float ps = 0.f;
        for (int i = 0; i < nr; ++i) {
            const float p = __builtin_amdgcn_exp2f(x[i] - m + kPShift);
            ps += p;
            phi[i] = (PE)p;
            plo[i] = (PE)(p - (float)phi[i]);
        }
        lp = fmaf(lp, corr, ps);
        if (rescale) {
            // O is held transposed (d rows 4*(l/16)+i of head l%16): the factor is in-lane
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                o[nb][0] *= corr; o[nb][1] *= corr; o[nb][2] *= corr; o[nb][3] *= corr;
            }
        }
    };

    // Step I for the 16-row tile at byte `kt` of the stage's K half: lane l gets the scores of
    // rows 4*(l/16)+i for head l%16.
    auto scores = [&](const char *kt, int t) {
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
        // line layout: this lane's row lr of the tile is row lr % 8 of piece 2t + lr / 8, and its
        // chunk 2 kb + lg / 2 sits at ((2 kb + lg / 2) ^ key) * 8 + lr % 8
        const char *kl = kt + (lr / 8) * 1024 + (lr % 8) * 16 + 8 * (lg % 2) +
                         (((lg / 2) ^ piece_key(2 * t + lr / 8)) << 7);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const uint2 v = kLines ? *reinterpret_cast<const uint2 *>(kl + kb * 256)
                                   : *reinterpret_cast<const uint2 *>(kt + ((kb * 2 + lg / 2) * 16 + lr) * 16 + 8 * (lg % 2));
            if constexpr (kF16)
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, i8x8_to_f16x8(v)),
                                                             __builtin_bit_cast(f16x8_t, qb[kb]), sacc, 0, 0, 0);
            else
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(v)),
                                                              __builtin_bit_cast(bf16x8_t, qb[kb]), sacc, 0, 0, 0);
        }
        return sacc;
    };

    auto process = [&](const char *st, int sb) {
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int blk = wb + j * WPH;  // P.V block of the stage
            const int rb = sb + blk * PVR; // its first cache row
            {
                // rows of lane group g: 4g+e (tile 0) and 16+4g+e (tile 1), e < 4
                const f32x4_t s0 = scores(st + (2 * blk) * TILE, 0);
                const f32x4_t s1 = scores(st + (2 * blk + 1) * TILE, 1);
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = (rb + 4 * lg + i < rend) ? s0[i] * scl : -INFINITY;
                    x[4 + i] = (rb + 16 + 4 * lg + i < rend) ? s1[i] * scl : -INFINITY;
                }
                PV phi, plo;
                softmax(x, phi, plo, 8);
                // V rows in the same order: lane s of group g reads row(g, s/2), bytes
                // 16*nb + 8*(s%2) .. +8; the transpose read hands lane l the 8 rows of column l%16.
                const int e = lr / 2;
                const int rr = e < 4 ? 4 * lg + e : 16 + 4 * lg + e - 4;
                const int vkey = piece_key(rr / 8);
                const char *vt = kLines ? st + HALF + (4 * blk + rr / 8) * 1024 + (rr % 8) * 16 + 8 * (lr % 2)
                                        : st + HALF + (2 * blk + rr / 16) * TILE + (rr % 16) * 16 + 8 * (lr % 2);
                // all hi products, then all lo ones (dependent MFMAs NB instructions apart)
                uint4 bvs[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int voff = kLines ? (nb ^ vkey) << 7 : nb * 256;
                    const auto t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) i32x2_t *)(lds_char *)(vt + voff));
                    const uint2 c8 = {(uint32_t)t[0], (uint32_t)t[1]};
                    if constexpr (kF16)
                        bvs[nb] = i8x8_to_f16x8(c8);
                    else
                        bvs[nb] = fp8x8_to_bf16x8(c8);
                }
                if constexpr (kF16) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, bvs[nb]), phi, o[nb], 0, 0, 0);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, bvs[nb]), plo, o[nb], 0, 0, 0);
                } else {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bvs[nb]), phi, o[nb], 0, 0, 0);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bvs[nb]), plo, o[nb], 0, 0, 0);
                }
            }
        }
    };

    // Stages alternate between s_a and s_b; before reading a stage each wave waits for its own
    // DMA into it (the other stage's may stay outstanding), then a barrier covers the others.
    const int nst = (r1 - r0 + RS - 1) / RS;
    issue(lds_a, r0);
    issue(lds_b, r0 + RS);
    for (int st = 0; st < nst; st += 2) {
        __builtin_amdgcn_s_waitcnt(vmcnt_only(VM_STAGE));
        __syncthreads();
        process(s_a, r0 + st * RS);
        __syncthreads();
        issue(lds_a, r0 + (st + 2) * RS);  // past the end this fetches nothing
        if (st + 1 < nst) {
            __builtin_amdgcn_s_waitcnt(vmcnt_only(VM_STAGE));
            __syncthreads();
            process(s_b, r0 + (st + 1) * RS);
            __syncthreads();
            issue(lds_b, r0 + (st + 3) * RS);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // no DMA into the stages is outstanding past this point

    // Merge: lane groups share each head's max (sums add); each wave puts its (max, sum) and O
    // into its own LDS slot (slots 0 and 1 in stage a, 2 and 3 in stage b). After one barrier
    // every thread merges float4 columns of the tile's rows over the slots of the waves that
    // hold the row's head tile (waves ht, ht + HT, ...) by their log-sum-exp weights and writes
    // them, so the outputs leave from all four waves at once. (The first version merged
    // pairwise: up to four barriers, one wave per head tile writing.)
    lp = xor32_sum(xor16_sum(lp));
    __syncthreads();
    // a slot: 16 rows of kRowO floats (a head's D outputs and a 16-byte pad: the 16 heads of a
    // wave's store fall on distinct banks)
    constexpr int kRowO = D + 4;
    static_assert(2 * 16 * kRowO * 4 <= 2 * HALF, "two merge slots per stage");
    auto mslot = [&](int w) { return reinterpret_cast<float *>(w < 2 ? s_a : s_b) + (w % 2) * 16 * kRowO; };
    if (lg == 0) { s_mm[wave][lr] = m; s_ll[wave][lr] = lp; }
    {
        float *so = mslot(wave);
        // O^T layout: lane l holds d = nb*16 + 4*(l/16) + i of head l%16
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            *reinterpret_cast<f32x4_t *>(&so[lr * kRowO + nb * 16 + 4 * lg]) = o[nb];
    }
    __syncthreads();
    constexpr int C4 = D / 4;  // float4 columns of a row
    for (int i = threadIdx.x; i < hv * C4; i += kBlock) {
        const int hd = i / C4, c4 = i % C4;
        const int t = hd / 16, hr = hd % 16;  // the row's head tile and its row in it
        float M = s_mm[t][hr];
        for (int w = t + HT; w < kWaves; w += HT) M = fmaxf(M, s_mm[w][hr]);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        float L = 0.f;
        for (int w = t; w < kWaves; w += HT) {
            const float f = __builtin_amdgcn_exp2f(s_mm[w][hr] - M);
            L = fmaf(s_ll[w][hr], f, L);
            const f32x4_t x = *reinterpret_cast<const f32x4_t *>(&mslot(w)[hr * kRowO + 4 * c4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(x[e], f, acc[e]);
        }
        const f32x4_t v = acc * vscale;
        if (direct) {
            const size_t row = query_row(a, b, kvh, h0, hd, slen).row;
            *reinterpret_cast<f32x4_t *>(&a.out[row * D + 4 * c4]) = v / L;
        } else {
            *reinterpret_cast<f32x4_t *>(&a.part_o[(k * a.gt + hd) * D + 4 * c4]) = v;
            if (c4 == 0) {
                a.part_ml[(k * a.gt + hd) * 2 + 0] = M - kPShift;
                a.part_ml[(k * a.gt + hd) * 2 + 1] = L;
            }
        }
    }
    __syncthreads();  // the LDS arrays are reused by the next segment
}

// Values read from LDS are per-lane to the compiler; the segment bounds are the same in every
// lane, and reading them through readfirstlane keeps them (and the buffer resources built from
// them) in scalar registers: a per-lane resource would wrap every buffer load in a loop.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The same 64-bit value from lane `lane` (uniform) of every lane.
__device__ __forceinline__ int64_t lane_value64(int64_t x, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)x, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)x >> 32), lane);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The segments of one workgroup, in order: rows [r0, r1) of (sequence sb, KV head kvh) for
// the hv query rows h0 .. h0+hv-1 of a head tile, partial slot k, whole = the segment is the
// entire unit. Every field but lane_len is the same in all lanes (scalar registers); copies of
// a walk advance independently.
// The walk finds its first row by the prefix over sequences of their rows; after that it needs
// only the stored lengths (a sequence has rows iff unit_rows of its length is non-zero). A batch
// of at most kWave sequences is held in lanes: every wave loads the lengths (lane b: sequence b)
// and scans them itself, with no LDS and no barrier; a larger one goes through LDS.
struct SegWalk {
    const int32_t *lens;  // the stored lengths in LDS, or null: lane_len holds them
    int32_t lane_len;     // lens[lane] in lanes < batch (a per-lane value)
    int64_t pos, end, w;
    int b, L, stored, ul, row, upb, g, gt, grp_rows, tiles, append_cap, max_len, nq;
    bool has;  // a current segment
    int sb, kvh, h0, hv, r0, r1;
    int slen;      // rows of the segment's sequence (the walk state moves on past them)
    size_t k;
    bool whole;
    bool new_row;  // this pass appended the unit's last row (row slen - 1)
    // An empty share (only when there are fewer rows than workgroups) whose position lies
    // strictly inside a unit: that unit's index (b * upb + ul), else -1. The combine reads
    // every workgroup between the unit's first and last, so this one leaves an empty partial.
    int64_t empty_unit;

    __device__ __forceinline__ int stored_len(int i) const {
        return lens ? __builtin_amdgcn_readfirstlane(lens[i]) : __builtin_amdgcn_readlane(lane_len, i);
    }
    __device__ __forceinline__ void init(const SplitArgs &a) {
        const Partition &pt = a.pt;
        gt = a.gt;
        grp_rows = a.grp_rows;
        tiles = pt.tiles;
        upb = pt.h_kv * pt.tiles;
        g = a.h_q / pt.h_kv;
        append_cap = pt.append_cap;
        max_len = pt.max_len;
        nq = pt.nq;
        w = blockIdx.x;
        b = 0, L = 1, stored = 0, ul = 0, row = 0;
        empty_unit = -1;
    }
    // Row `pos` lies in sequence b0, whose rows start at position pre_b (b0 has rows).
    __device__ __forceinline__ void locate(int b0, int64_t pre_b) {
        b = b0;
        stored = stored_len(b);
        L = attended_len(stored, append_cap);
        const int64_t off = pos - pre_b;
        ul = (int)(off / L);  // unit within the sequence
        row = (int)(off % L);
        if (pos == end && row > 0) empty_unit = (int64_t)b * upb + ul;
    }
    // Positions the walk on the workgroup's first segment; s_pre must hold the prefix and
    // s_len the stored lengths.
    __device__ __forceinline__ void start(const SplitArgs &a, const int64_t *s_pre, const int32_t *s_len) {
        init(a);
        lens = s_len;
        const int64_t Tot = uniform64(s_pre[a.pt.batch]), N = a.pt.nwg;
        pos = wg_start(w, Tot, N);
        end = wg_start(w + 1, Tot, N);
        if (pos < Tot) {
            // the sequence holding row `pos`: the last b with pre[b] <= pos (it has rows)
            int lo = 0, hi = a.pt.batch;  // invariant: pre[lo] <= pos < pre[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) / 2;
                if (uniform64(s_pre[mid]) <= pos) lo = mid; else hi = mid;
            }
            locate(lo, uniform64(s_pre[lo]));
        }
        next();
    }
    // The same for a batch of at most kWave sequences, from the lengths in memory.
    __device__ __forceinline__ void start_in_lanes(const SplitArgs &a) {
        init(a);
        lens = nullptr;
        const Partition &pt = a.pt;
        const int lane = threadIdx.x % kWave;
        lane_len = lane < pt.batch ? a.lens[lane] : 0;
        const int64_t own =
            lane < pt.batch ? unit_rows(attended_len(lane_len, append_cap), max_len, nq) * upb : 0;
        int64_t incl = own;
#pragma unroll
        for (int off = 1; off < kWave; off *= 2) {
            const int64_t y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        const int64_t excl = incl - own;
        const int64_t Tot = lane_value64(incl, kWave - 1), N = pt.nwg;
        pos = wg_start(w, Tot, N);
        end = wg_start(w + 1, Tot, N);
        if (pos < Tot) {
            // the lanes with pre[b] <= pos are a prefix (lane 0 among them): the last one
            const uint64_t m = __ballot(excl <= pos);
            const int b0 = 63 - __builtin_clzll(m);
            locate(b0, lane_value64(excl, b0));
        }
        next();
    }
    __device__ __forceinline__ void next() {
        has = pos < end;
        if (!has) return;
        r0 = row;
        r1 = (int)min<int64_t>((int64_t)L, row + (end - pos));
        kvh = ul / tiles;
        h0 = kvh * g + (ul % tiles) * gt;
        hv = min(gt, grp_rows - (ul % tiles) * gt);
        sb = b;
        k = (size_t)w + (size_t)b * upb + ul;
        slen = L;
        whole = r0 == 0 && r1 == L;
        new_row = append_cap > 0 && L != stored;
        pos += r1 - r0;
        row = 0;
        if (++ul == upb && pos < end) {
            ul = 0;
            do {  // skip sequences without rows
                ++b;
                stored = stored_len(b);
                L = attended_len(stored, append_cap);
            } while (unit_rows(L, max_len, nq) == 0);
        }
    }
};

// Computes the sequence prefix (in lanes, or in LDS) and returns the walk on the workgroup's
// first segment.
__device__ __forceinline__ SegWalk first_segment(const SplitArgs &a) {
    __shared__ int64_t s_pre[kMaxBatch + 1];
    __shared__ int64_t s_wave[kWaves];
    __shared__ int32_t s_len[kMaxBatch];
    if (a.pt.append_cap > 0 && blockIdx.x == 0) {
        // the combine reads the stored lengths from this copy, so that it may update lens
        for (int b = threadIdx.x; b < a.pt.batch; b += kBlock) {
            const int L = a.lens[b];
            a.lens_copy[b] = L;
            if (L < 0 || L >= a.pt.append_cap) atomicOr(a.err, DA_DEV_ERR_APPEND_FULL);
        }
    }
    SegWalk wk;
    if (a.pt.batch <= kWave) {
        wk.start_in_lanes(a);
    } else {
        sequence_prefix(a.lens, a.pt, s_pre, s_wave, s_len);
        wk.start(a, s_pre, s_len);
    }
    return wk;
}

// Workgroup w walks its share of the rows and calls seg(b, kvh, h0, hv, r0, r1, k, whole, slen)
// once per unit it crosses. The workgroup holding a unit's first row, and the one holding its last,
// record themselves in the unit's entry of unit_wg, so that the combine finds the unit's
// segments without redoing the partition.
// With a fused append, a segment that ends at a unit's new last row first stores that row of
// K and V into the cache itself; the barrier (a workgroup-scope release and acquire) makes the
// stores visible to the loads of every wave of the workgroup. Only workgroups holding that
// row read it in this pass, and each of them writes it (the same bytes) before reading.
template <class SegFn>
__device__ __forceinline__ void walk_segments(const SplitArgs &a, SegFn &&seg) {
    SegWalk wk = first_segment(a);
    if (wk.empty_unit >= 0) {  // (max, sum, row) = (kNegBig, 0, 0): weighs nothing in the combine
        const size_t kk = (size_t)wk.w + (size_t)wk.empty_unit;
        const int gt = a.gt;
        for (int i = threadIdx.x; i < gt * 2; i += kBlock) a.part_ml[kk * gt * 2 + i] = (i % 2) ? 0.f : kNegBig;
        for (int i = threadIdx.x; i < gt * a.dv; i += kBlock) a.part_o[kk * gt * a.dv + i] = 0.f;
    }
    for (; wk.has; wk.next()) {
        if (wk.new_row && wk.r1 == wk.slen) {
            const int n16 = a.row_bytes / 16;
            const size_t slot = (size_t)wk.sb * a.pt.h_kv + wk.kvh;
            const int t = threadIdx.x;
            if (t < 2 * n16) {
                const bool v = t >= n16;
                const uint4 x = reinterpret_cast<const uint4 *>(
                    static_cast<const char *>(v ? a.v_new : a.k_new) + slot * a.row_bytes)[t % n16];
                char *dst = const_cast<char *>(static_cast<const char *>(v ? a.vc : a.kc)) +
                            (slot * a.cap + (wk.slen - 1)) * (size_t)a.row_bytes;
                reinterpret_cast<uint4 *>(dst)[t % n16] = x;
            }
            __syncthreads();
            // A row that does not fill whole cache lines shares a line with the previous row,
            // which another workgroup on this CU may hold, stale, in the vector L1: drop it.
            // Rows of whole lines need nothing: no workgroup reads a new row's lines in this
            // pass before storing them itself (the agent-scope acquire also costs the whole
            // workgroup its L2 round trips: 6 us of an 8K-row GQA step).
            if (a.shared_lines) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        if (threadIdx.x == 0) {
            int32_t *uw = reinterpret_cast<int32_t *>(a.unit_wg + (wk.k - wk.w));
            if (wk.r0 == 0) uw[0] = (int32_t)wk.w;
            if (wk.r1 == wk.slen) uw[1] = (int32_t)wk.w;
        }
        seg(wk.sb, wk.kvh, wk.h0, wk.hv, wk.r0, wk.r1, wk.k, wk.whole, wk.slen);
    }
}

// VALU flavour (GT = 1, 2, 4 or 8 query-row slots, of which a tile's hv are live). DIRECT
// (decode_attn_run): a unit covered by a single workgroup is written to out directly and
// lse_combine_kernel skips it; otherwise every segment leaves a partial result.
template <int KV, int D, int GT, bool DIRECT>
__global__ __launch_bounds__(kBlock) void split_kv_attn_kernel(const SplitArgs a) {
    walk_segments(a, [&](int b, int kvh, int h0, int hv, int r0, int r1, size_t k, bool whole, int slen) {
        attend_segment<KV, D, GT>(a, b, kvh, h0, hv, r0, r1, k, DIRECT && whole, slen);
    });
}

// Matrix-core flavour (GW = 16 or 32 query-row slots; bf16, fp8 or int8 caches): bf16 streams
// through the register ring, 8-bit caches through the LDS stages.
// Register targets: 16 slots are held to 256 registers so that two waves fit per SIMD; 32 slots
// may use the whole register file (d = 128 bf16 comes out at 256 vector registers and a few
// accumulation registers, one wave per SIMD; the plan gives that kernel one workgroup per CU in
// any case: two measured slower).
template <int GW>
struct MfmaWaves { static constexpr int kMin = GW == 32 ? 1 : 2; };

// Register ring depth of the bf16 matrix-core segment (tiles of 16 rows per wave); deeper
// rings measured no faster and need more registers.
constexpr int kMfmaRing = 2;

template <int KV, int D, int GW, bool DIRECT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(MfmaWaves<GW>::kMin)))
void split_kv_attn_mfma_kernel(const SplitArgs a) {
    if constexpr (Kv<KV>::kEsz == 1) {
        walk_segments(a, [&](int b, int kvh, int h0, int hv, int r0, int r1, size_t k, bool whole, int slen) {
            attend_segment_staged<KV, D, GW>(a, b, kvh, h0, hv, r0, r1, k, DIRECT && whole, slen);
        });
    } else {
        walk_segments(a, [&](int b, int kvh, int h0, int hv, int r0, int r1, size_t k, bool whole, int slen) {
            attend_segment_mfma<KV, D, GW, kMfmaRing>(a, b, kvh, h0, hv, r0, r1, k, DIRECT && whole, slen);
        });
    }
}

// Single pass (one launch), for latency-bound problems. Workgroup x takes split s of unit ul of
// sequence b (x = (b * units + ul) * nsplit + s; a unit is a (KV head, head tile) as in the
// split path, here on the vector ALUs): rows [s * n / nsplit, (s + 1) * n / nsplit) of the
// sequence's n rows. With an append the workgroup whose rows end at the new last row stores it
// first (as in the split path). Each split leaves its partial result, written through to the
// device's coherence point (agent-scope stores), and counts itself in the unit's counter; the
// split that arrives last merges the unit's partials by their log-sum-exp weights and writes out.
// The order stores -> counter -> loads is made by the hardware's own means: every thread waits
// for its stores to complete (vmcnt) before the barrier that precedes the counter's atomic add,
// and the merging workgroup reads the partials with agent-scope loads, issued after its own
// add returned. No workgroup ever waits for another, so no launch order or residency is
// assumed. Every workgroup of a sequence also counts itself in the sequence's counter once it
// has read lens[b]; the last of them advances lens[b] (with an append), when no workgroup of the
// launch will read it again. Counters rest at zero: the last arrival resets each one.
constexpr int kMaxSingleSplits = 64;

template <int KV, int D, int GT>
__global__ __launch_bounds__(kBlock) void decode_step_single_kernel(const SplitArgs a) {
    const int S = a.nsplit, upb = a.pt.h_kv * a.pt.tiles;
    const int x = blockIdx.x;
    const int b = x / (upb * S), ul = (x / S) % upb, s = x % S;
    const int kvh = ul / a.pt.tiles, t = ul % a.pt.tiles;
    const int g = a.h_q / a.pt.h_kv;
    const int h0 = kvh * g + t * a.gt, hv = min(a.gt, a.grp_rows - t * a.gt);
    const bool append = a.pt.append_cap > 0;
    // lens[b] is read by thread 0 alone and handed to the others through LDS, so that it is
    // certainly read before this workgroup counts itself in the sequence's counter
    __shared__ int s_len, s_last;
    if (threadIdx.x == 0) s_len = a.lens[b];
    __syncthreads();
    const int L = s_len;
    const int n = attended_len(L, append ? a.pt.append_cap : 0);
    // count this workgroup in the sequence's counter now (lens[b] is read); the answer is only
    // looked at when the workgroup ends, so the atomic's round trip overlaps the attention
    int seq_arrived = 0;
    if (threadIdx.x == 0) {
        if (append && n == L && ul == 0 && s == 0) atomicOr(a.err, DA_DEV_ERR_APPEND_FULL);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        seq_arrived = __hip_atomic_fetch_add(&a.seq_cnt[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the last of the sequence's workgroups to count itself advances lens[b]: every workgroup of
    // the launch that reads it has read it
    auto finish_sequence = [&]() {
        if (threadIdx.x == 0 && seq_arrived == upb * S - 1) {
            __hip_atomic_store(&a.seq_cnt[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (append && n != L) a.lens[b] = n;
        }
    };
    const size_t slot = (size_t)b * upb + ul;  // the unit's index
    if (unit_rows(n, a.pt.max_len, a.pt.nq) == 0) {
        if (s == 0) {  // this unit's query rows are zeroed
            for (int i = threadIdx.x; i < hv * D; i += kBlock)
                a.out[query_row(a, b, kvh, h0, i / D, n).row * D + i % D] = 0.f;
            if (threadIdx.x == 0) atomicOr(a.err, DA_DEV_ERR_LEN_RANGE);
        }
        finish_sequence();
        return;
    }
    const int r0 = (int)((int64_t)s * n / S), r1 = (int)((int64_t)(s + 1) * n / S);
    if (append && n != L && r1 == n) {
        const int n16 = a.row_bytes / 16;
        const size_t kv = (size_t)b * a.pt.h_kv + kvh;
        if (threadIdx.x < 2 * n16) {
            const bool v = threadIdx.x >= n16;
            const int j = threadIdx.x % n16;
            const uint4 y = reinterpret_cast<const uint4 *>(static_cast<const char *>(v ? a.v_new : a.k_new) +
                                                            kv * a.row_bytes)[j];
            char *dst = const_cast<char *>(static_cast<const char *>(v ? a.vc : a.kc)) +
                        (kv * a.cap + L) * (size_t)a.row_bytes;
            reinterpret_cast<uint4 *>(dst)[j] = y;
        }
        __syncthreads();
        // a row shorter than a cache line shares its line with the previous row, which another
        // workgroup on this CU may hold, stale, in the vector L1: drop it
        if (a.shared_lines) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    if (S == 1) {  // the whole unit: normalised straight to out
        attend_segment<KV, D, GT>(a, b, kvh, h0, hv, 0, n, 0, true, n);
        finish_sequence();
        return;
    }
    const size_t k = slot * S + s;
    attend_segment<KV, D, GT, kWaves, kUnroll, true>(a, b, kvh, h0, hv, r0, r1, k, false, n);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const int arrived = __hip_atomic_fetch_add(&a.unit_cnt[slot], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = arrived == S - 1;
        if (s_last) __hip_atomic_store(&a.unit_cnt[slot], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    finish_sequence();
    if (!s_last) return;
    // The last split of the unit merges the nsplit partials of each of its hv query rows. Each
    // (row, column) item takes tp threads (consecutive lanes, as many as 256 threads give each
    // item, at most 8), each of which loads its share of the splits in one batch and keeps a
    // running maximum; the tp threads then merge by lane exchanges. The partials are read with
    // agent-scope (sc1) buffer loads, which the coherence point serves, and which, unlike atomic
    // loads, the compiler issues together.
    constexpr int kSc1 = 16;  // cache-policy bit of an agent-scope access
    const __amdgpu_buffer_rsrc_t mls = make_rsrc(a.part_ml + slot * S * a.gt * 2, (uint32_t)(S * a.gt * 2 * 4));
    const __amdgpu_buffer_rsrc_t os = make_rsrc(a.part_o + slot * S * a.gt * D, (uint32_t)(S * a.gt * D * 4));
    const int items = hv * D;
    const int tp = items >= kBlock / 2 ? 1 : items >= kBlock / 4 ? 2 : items >= kBlock / 8 ? 4 : 8;
    for (int i0 = 0; i0 < items * tp; i0 += kBlock) {
        const int i = (i0 + (int)threadIdx.x) / tp, sub = (i0 + (int)threadIdx.x) % tp;
        const int h = min(i, items - 1) / D, d = min(i, items - 1) % D;
        float M = kNegBig, Z = 0.f, O = 0.f;
        for (int j0 = sub; j0 < S; j0 += 8 * tp) {
            float mj[8], lj[8], oj[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {  // splits past nsplit are past the resources: zeros
                const uint32_t kk = (uint32_t)((j0 + u * tp) * a.gt + h);
                mj[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mls, kk * 8, 0, kSc1));
                lj[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mls, kk * 8 + 4, 0, kSc1));
                oj[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(os, (kk * D + d) * 4, 0, kSc1));
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u * tp >= S) break;
                const float Mn = fmaxf(M, mj[u]);
                const float c = __builtin_amdgcn_exp2f(M - Mn), f = __builtin_amdgcn_exp2f(mj[u] - Mn);
                Z = fmaf(Z, c, lj[u] * f);
                O = fmaf(O, c, oj[u] * f);
                M = Mn;
            }
        }
        for (int off = 1; off < tp; off *= 2) {  // the item's tp lanes are consecutive
            const float Mo = __shfl_xor(M, off), Zo = __shfl_xor(Z, off), Oo = __shfl_xor(O, off);
            const float Mn = fmaxf(M, Mo);
            const float c = __builtin_amdgcn_exp2f(M - Mn), f = __builtin_amdgcn_exp2f(Mo - Mn);
            Z = fmaf(Z, c, Zo * f);
            O = fmaf(O, c, Oo * f);
            M = Mn;
        }
        if (sub == 0 && i < items) a.out[query_row(a, b, kvh, h0, h, n).row * D + d] = O / Z;
    }
}

// Merges the segments of every query row by their log-sum-exp weights. Workgroup x takes
// column slice x % cs (D / cs columns) of rows rw * (x / cs % (gt / rw)) .. + rw - 1 of unit
// u = x / cs / (gt / rw) (a unit's rows share its segments), each row with kCombineBlock / rw
// threads: segment groups of D / (4 cs) threads, one float4 column each. Column slices spread a
// few rows with many segments (MQA: 4 units, 64 segments a row) over more workgroups. The
// last head tile of a group may hold fewer than gt rows (grp_rows, the group's g * nq query
// rows, need not be a multiple of gt): the rows past it are merged from slots nothing wrote and
// not stored. skip_single: a unit covered by one workgroup was already written.
// With a fused append (pt.append_cap > 0) the stored lengths come from the split kernel's
// workspace copy, and the workgroup of head 0 writes each sequence's new length to lens_upd.
// The unit's segments are those of workgroups unit_wg[u].x .. unit_wg[u].y (slot w + u), which
// the split kernel recorded; every workgroup in between left a partial for the unit (an empty
// one if its share holds no rows). The length and that entry are read together, then every
// segment once: each segment group keeps a running maximum; the groups of a row merge by
// shuffles within a wave, then the waves of a row through LDS.
// lse_out (decode_attn_run_lse; NULL otherwise): each row's log-sum-exp of its scaled scores,
// natural log, ln sum_l exp(s[l]) = ln 2 * (M + log2 l) for the merged base-2 maximum M and
// sum l, so that results over disjoint row sets merge by decode_attn_merge_lse. In this mode a
// sequence of length 0 holds no rows of this shard: output 0 and log-sum-exp -inf, no error.
template <int D>
__global__ __launch_bounds__(kCombineBlock) void lse_combine_kernel(
    const int32_t *__restrict__ lens, int32_t *__restrict__ lens_upd, const int2 *__restrict__ unit_wg,
    const float *__restrict__ part_ml, const float *__restrict__ part_o,
    float *__restrict__ out, int32_t *__restrict__ err, int h_q, int gt, int grp_rows, int rw, int cs,
    Partition pt, int skip_single, float *__restrict__ lse_out) {
    constexpr int UN = 8;          // segments a group loads before using them
    const int cw = D / 4 / cs;     // float4 columns of the slice
    const int tpr = kCombineBlock / rw, sgr = tpr / cw;  // threads and segment groups per row
    const int per_unit = gt / rw;
    const int xs = blockIdx.x / cs;
    const int64_t u = xs / per_unit;
    const int hh = (xs % per_unit) * rw + threadIdx.x / tpr;  // the thread's row in the unit
    const int sg = threadIdx.x % tpr / cw;
    const int c4 = (blockIdx.x % cs) * cw + threadIdx.x % cw;  // the thread's float4 column
    const int upb = pt.h_kv * pt.tiles, g = h_q / pt.h_kv;
    const int b = (int)(u / upb), ul = (int)(u % upb), kvh = ul / pt.tiles;
    // the row's query position and head: row hh of the tile is row fr of the group's g * nq
    const int fr = (ul % pt.tiles) * gt + hh, tq = fr / g, h = kvh * g + fr % g;
    const bool live = fr < grp_rows;  // a query row of the group, not past its last tile's rows
    const size_t orow = (size_t)(b * pt.nq + tq) * h_q + h;
    float *dst = out + orow * D;
    const int L = attended_len(lens[b], pt.append_cap);
    const int2 ww = unit_wg[u];
    if (lens_upd && ul == 0 && threadIdx.x == 0 && xs % per_unit == 0 && blockIdx.x % cs == 0) lens_upd[b] = L;
    if (unit_rows(L, pt.max_len, pt.nq) == 0) {
        if (sg == 0 && live) {
            reinterpret_cast<float4 *>(dst)[c4] = float4{0.f, 0.f, 0.f, 0.f};
            if (lse_out && c4 == 0) lse_out[orow] = -INFINITY;
        }
        if (threadIdx.x == 0 && !(lse_out && L == 0)) atomicOr(err, DA_DEV_ERR_LEN_RANGE);
        return;
    }
    const int wa = ww.x, wb = ww.y;
    if (skip_single && wa == wb) return;

    float4 acc = {0.f, 0.f, 0.f, 0.f};
    float mrun = kNegBig, ls = 0.f;  // an absent segment is (kNegBig, 0, 0): weight 0 or no effect
    for (int w0 = wa + sg; w0 <= wb; w0 += sgr * UN) {
        float2 mlj[UN];
        float4 oj[UN];
#pragma unroll
        for (int j = 0; j < UN; ++j) {
            const int w = w0 + j * sgr;
            mlj[j] = float2{kNegBig, 0.f};
            oj[j] = float4{0.f, 0.f, 0.f, 0.f};
            if (w <= wb) {
                const size_t kk = (size_t)(w + u) * gt + hh;
                mlj[j] = reinterpret_cast<const float2 *>(part_ml)[kk];
                oj[j] = reinterpret_cast<const float4 *>(part_o + kk * D)[c4];
            }
        }
        float mx = mrun;
#pragma unroll
        for (int j = 0; j < UN; ++j) mx = fmaxf(mx, mlj[j].x);
        const float r = __builtin_amdgcn_exp2f(mrun - mx);
        ls *= r;
        acc.x *= r;
        acc.y *= r;
        acc.z *= r;
        acc.w *= r;
#pragma unroll
        for (int j = 0; j < UN; ++j) {
            const float f = __builtin_amdgcn_exp2f(mlj[j].x - mx);
            ls = fmaf(mlj[j].y, f, ls);
            acc.x = fmaf(oj[j].x, f, acc.x);
            acc.y = fmaf(oj[j].y, f, acc.y);
            acc.z = fmaf(oj[j].z, f, acc.z);
            acc.w = fmaf(oj[j].w, f, acc.w);
        }
        mrun = mx;
    }
    // (M, l, o) of two groups -> their merge, for a partner `off` lanes away
    auto merge_with = [&](int off) {
        const float Mo = __shfl_xor(mrun, off), lo = __shfl_xor(ls, off);
        const float ox = __shfl_xor(acc.x, off), oy = __shfl_xor(acc.y, off);
        const float oz = __shfl_xor(acc.z, off), ow = __shfl_xor(acc.w, off);
        const float M = fmaxf(mrun, Mo);
        const float f = __builtin_amdgcn_exp2f(mrun - M), fo = __builtin_amdgcn_exp2f(Mo - M);
        ls = fmaf(ls, f, lo * fo);
        acc = float4{fmaf(acc.x, f, ox * fo), fmaf(acc.y, f, oy * fo), fmaf(acc.z, f, oz * fo), fmaf(acc.w, f, ow * fo)};
        mrun = M;
    };
    // the groups of a row within a wave sit cw, 2 cw, ... lanes apart
    const int span = tpr < kWave ? tpr : kWave;  // lanes of one row within a wave
    for (int off = cw; off < span; off *= 2) merge_with(off);
    constexpr int kCombineWaves = kCombineBlock / kWave;
    __shared__ float4 s_acc[kCombineWaves][kWave];
    __shared__ float s_m[kCombineWaves], s_l[kCombineWaves];
    const int wpr = tpr / kWave;  // waves per row (0: several rows per wave, merged already)
    if (wpr > 1) {
        const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
        if (lane < cw) {
            s_acc[wave][lane] = acc;
            if (lane == 0) { s_m[wave] = mrun; s_l[wave] = ls; }
        }
        __syncthreads();
        if (wave % wpr != 0 || lane >= cw) return;  // the row's first wave finishes it
        float M = s_m[wave];
        for (int i = 1; i < wpr; ++i) M = fmaxf(M, s_m[wave + i]);
        float4 x = {0.f, 0.f, 0.f, 0.f};
        float z = 0.f;
        for (int i = 0; i < wpr; ++i) {
            const float f = __builtin_amdgcn_exp2f(s_m[wave + i] - M);
            const float4 y = s_acc[wave + i][lane];
            x.x = fmaf(y.x, f, x.x);
            x.y = fmaf(y.y, f, x.y);
            x.z = fmaf(y.z, f, x.z);
            x.w = fmaf(y.w, f, x.w);
            z = fmaf(s_l[wave + i], f, z);
        }
        acc = x;
        ls = z;
        mrun = M;
    } else if (sg != 0) {
        return;
    }
    if (live) {
        reinterpret_cast<float4 *>(dst)[c4] = float4{acc.x / ls, acc.y / ls, acc.z / ls, acc.w / ls};
        if (lse_out && c4 == 0) lse_out[orow] = (mrun + __log2f(ls)) * kLn2;
    }
}

// Log-sum-exp merge of `shards` results over disjoint row sets (decode_attn_merge_lse): thread
// x takes float4 column x % (d / 4) of row x / (d / 4). With M = max_p lse_p and
// w_p = exp(lse_p - M): out = sum_p w_p out_p / sum_p w_p and lse = M + ln sum_p w_p, Step II's
// normalisation over the union of the shards' rows. A row that no shard holds (every lse_p
// -inf) gets out 0 and lse -inf.
__global__ __launch_bounds__(256) void merge_lse_kernel(int64_t rows, int d, int shards, const float *__restrict__ outs,
                                                        const float *__restrict__ lses, float *__restrict__ out,
                                                        float *__restrict__ lse_out) {
    const int c4n = d / 4;
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= rows * c4n) return;
    const int64_t r = x / c4n;
    const int c4 = (int)(x % c4n);
    float M = -INFINITY;
    for (int p = 0; p < shards; ++p) M = fmaxf(M, lses[p * rows + r]);
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    float z = 0.f;
    if (M != -INFINITY) {
        for (int p = 0; p < shards; ++p) {
            const float w = __builtin_amdgcn_exp2f((lses[p * rows + r] - M) * kLog2e);
            const float4 o = reinterpret_cast<const float4 *>(outs + ((size_t)p * rows + r) * d)[c4];
            z += w;
            acc.x = fmaf(o.x, w, acc.x);
            acc.y = fmaf(o.y, w, acc.y);
            acc.z = fmaf(o.z, w, acc.z);
            acc.w = fmaf(o.w, w, acc.w);
        }
        acc = float4{acc.x / z, acc.y / z, acc.z / z, acc.w / z};
    }
    reinterpret_cast<float4 *>(out + (size_t)r * d)[c4] = acc;
    if (lse_out && c4 == 0) lse_out[r] = M == -INFINITY ? M : M + __logf(z);
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

int elem_size(int dt) {
    return dt == DA_F32 ? 4 : dt == DA_BF16 ? 2 : (dt == DA_FP8_E4M3FN || dt == DA_INT8) ? 1 : 0;
}

int validate(const da_desc *d) {
    if (!d) return fail(DA_ERR_INVALID_ARG, "desc is NULL");
    if (d->batch < 1 || d->h_q < 1 || d->h_kv < 1 || d->cap < 1 || d->d_k < 1 || d->d_v < 1)
        return fail(DA_ERR_INVALID_ARG, "batch, heads, head sizes and cap must be positive");
    if (d->batch > kMaxBatch)
        return fail(DA_ERR_UNSUPPORTED, "batch is limited to %d sequences per call (got %d)", kMaxBatch, d->batch);
    if (d->h_q % d->h_kv)
        return fail(DA_ERR_INVALID_ARG, "h_q (%d) is not a multiple of h_kv (%d)", d->h_q, d->h_kv);
    if (!std::isfinite(d->scale)) return fail(DA_ERR_INVALID_ARG, "scale is not finite");
    if (d->block_rows < 0) return fail(DA_ERR_INVALID_ARG, "block_rows must be >= 0");
    if (!elem_size(d->q_dtype) || !elem_size(d->kv_dtype))
        return fail(DA_ERR_INVALID_ARG, "unknown dtype code");
    if (d->d_k != d->d_v || (d->d_k != 64 && d->d_k != 128))
        return fail(DA_ERR_UNSUPPORTED, "head sizes d_k = d_v in {64, 128} are supported (got %d, %d)",
                    d->d_k, d->d_v);
    const bool ok = (d->q_dtype == DA_F32 && d->kv_dtype == DA_F32) ||
                    (d->q_dtype == DA_BF16 && d->kv_dtype == DA_BF16) ||
                    (d->q_dtype == DA_BF16 && d->kv_dtype == DA_FP8_E4M3FN) ||
                    (d->q_dtype == DA_BF16 && d->kv_dtype == DA_INT8);
    if (!ok) return fail(DA_ERR_UNSUPPORTED, "dtype pair (q %d, kv %d) is not built", d->q_dtype, d->kv_dtype);
    if (d->path != DA_PATH_AUTO && d->path != DA_PATH_SPLIT && d->path != DA_PATH_SINGLE)
        return fail(DA_ERR_INVALID_ARG, "path must be DA_PATH_AUTO, _SPLIT or _SINGLE (got %d)", d->path);
    if (d->path == DA_PATH_SINGLE && d->block_rows)
        return fail(DA_ERR_INVALID_ARG, "block_rows sizes the split path's shares: it must be 0 with DA_PATH_SINGLE");
    if (d->flavour != DA_FLAVOUR_AUTO && d->flavour != DA_FLAVOUR_VECTOR && d->flavour != DA_FLAVOUR_MATRIX)
        return fail(DA_ERR_INVALID_ARG, "flavour must be DA_FLAVOUR_AUTO, _VECTOR or _MATRIX (got %d)", d->flavour);
    if (d->n_queries < 0 || d->n_queries > kMaxQueries)
        return fail(DA_ERR_INVALID_ARG, "n_queries must be in [0, %d] (got %d)", kMaxQueries, d->n_queries);
    return DA_OK;
}

// Query rows per sequence (0 and 1 both mean single-query decode), and per KV group.
int n_queries(const da_desc *d) { return d->n_queries > 1 ? d->n_queries : 1; }
int group_rows(const da_desc *d) { return d->h_q / d->h_kv * n_queries(d); }

// Workspace layout, each section starting on a 256-byte boundary: [error word, padded to
// 256 B][copy of the stored lengths, batch int32 (fused append)][the single pass's arrival
// counters, batch + its units int32][per unit, its first and last workgroup, int2][partial
// (max, sum) pairs, 2 fp32 a row][partial output rows, d_v fp32 a row]. The partial arrays
// hold (N + units) * GT rows for the split path (N workgroups, units = batch * h_kv * head
// tiles), or the single pass's units * nsplit * GT, whichever is larger.
struct Plan {
    int gt;     // query rows per head tile (the last tile of a group may hold fewer)
    int gw;     // the kernel's query-row slots, >= gt (slots past a tile's rows are padding)
    int tiles;  // head tiles per KV group
    int nwg;
    bool mfma;  // matrix-core flavour
    // one-call entry points: the single pass (one launch, splits merged by the last to finish)
    // instead of the split kernel and the combine; its tiling (vector ALUs) replaces
    // gt / gw / tiles when set
    bool single;
    int nsplit;      // single pass: splits per unit
    size_t cnt_off;  // single pass: arrival counters, per sequence then per unit
    size_t ncnt;     // single pass: counters (batch + units)
    // workspace offsets: lengths copy, per-unit first / last workgroup, (max, sum), rows; total
    size_t lens_off, unit_off, ml_off, o_off, bytes;
};

// Flavour and head tiles. A KV group's g * T query rows (T query rows per sequence) read each K
// and V row once per head tile, so a group is cut into as few tiles as the flavour's widest
// workgroup allows, of nearly equal size, and each tile is padded up to the kernel's slot
// count with zero queries instead of being split further:
//   * bf16 / fp8 / int8 caches with at least 3 query rows per group run on the matrix cores,
//     tiles of up to 32 rows in 16 or 32 slots (one tile, one read of the group's rows, for
//     every g * T <= 32);
//   * otherwise the vector ALUs: fp32 caches with tiles of up to 8 rows, 8-bit and bf16 caches
//     with 1 or 2 rows (up to 4 when the vector ALUs are asked for), in 1, 2, 4 or 8 slots.
// desc->flavour asks for one flavour (measurement: both flavours on one shape).
int plan_tiles(const da_desc *d, Plan *p, bool vector_only = false) {
    const int rows = group_rows(d);
    const bool can_mfma = d->kv_dtype != DA_F32 && !vector_only;
    if (d->flavour == DA_FLAVOUR_MATRIX && !can_mfma)
        return fail(DA_ERR_UNSUPPORTED, vector_only ? "the single pass runs on the vector ALUs only"
                                                    : "the matrix-core flavour takes bf16, fp8 or int8 caches");
    p->mfma = d->flavour == DA_FLAVOUR_MATRIX || (d->flavour == DA_FLAVOUR_AUTO && can_mfma && rows >= 3);
    const int widest = p->mfma ? 32 : d->kv_dtype == DA_F32 ? 8 : 4;
    p->tiles = (rows + widest - 1) / widest;
    p->gt = (rows + p->tiles - 1) / p->tiles;
    if (p->mfma) p->gw = p->gt <= 16 ? 16 : 32;
    else p->gw = p->gt <= 1 ? 1 : p->gt <= 2 ? 2 : p->gt <= 4 ? 4 : 8;
    return DA_OK;
}

// Bytes past a segment's last row that prefetches may address (LDS stages run up to four 16 KiB
// stages ahead; register rings one 64-row step of 512-byte rows); kept well above that.
constexpr int64_t kSlotSlack = int64_t(1) << 20;
constexpr int kMinRowsPerBlock = 256;  // below this a workgroup's share is mostly overhead
// The library's choice of the single pass for the one-call entry points: every sequence's K and
// V bytes at max_len (all its head tiles) at most this.
constexpr int64_t kSingleMaxBytes = int64_t(1) << 20;
// Rows per split of the single pass at max_len (each unit is cut into ceil(max_len / kSingleRows)
// splits, at most kMaxSingleSplits): one 64-row step of a 4-wave workgroup.
constexpr int kSingleRows = 64;
constexpr int kFallbackResident = 512; // workgroups planned for when no device is visible

// Workgroups to launch for one split-kernel instantiation on the current device: every CU
// gets the same number, min(what fits, the cap), cached per (device, kernel). Measured on
// MI355X (256 CUs), counts that are not a multiple of the CU count leave some CUs with more
// shares than others and run up to 15 % slower; two 4-wave workgroups per CU stream faster
// than three. The bf16 register ring with 32 slots is capped at one per CU: two (the ring held
// to 252 registers, so that two fit per SIMD) took MQA from 48 to 53 us.
constexpr int kBlocksPerCu = 2;
// Compute units of the current device (256 when it cannot be queried).
int cu_count() {
    static std::mutex mu;
    static std::map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
        (void)hipGetLastError();
        return 256;
    }
    return cache[dev] = cus;
}

int resident_workgroups(const void *kernel, int max_per_cu) {
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return kFallbackResident / kBlocksPerCu * max_per_cu;
    }
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({dev, kernel});
    if (it != cache.end()) return it->second;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0) != hipSuccess || cus < 1 ||
        per_cu < 1) {
        (void)hipGetLastError();
        return kFallbackResident / kBlocksPerCu * max_per_cu;
    }
    return cache[{dev, kernel}] = cus * std::min(per_cu, max_per_cu);
}

template <int KV, int D>
const void *split_kernel_ptr(int gw, bool mfma) {
    if constexpr (KV != DA_F32) {
        if (mfma)
            return gw == 32 ? reinterpret_cast<const void *>(&split_kv_attn_mfma_kernel<KV, D, 32, false>)
                            : reinterpret_cast<const void *>(&split_kv_attn_mfma_kernel<KV, D, 16, false>);
    } else {
        if (gw == 8) return reinterpret_cast<const void *>(&split_kv_attn_kernel<KV, D, 8, false>);
    }
    switch (gw) {
    case 4: return reinterpret_cast<const void *>(&split_kv_attn_kernel<KV, D, 4, false>);
    case 2: return reinterpret_cast<const void *>(&split_kv_attn_kernel<KV, D, 2, false>);
    default: return reinterpret_cast<const void *>(&split_kv_attn_kernel<KV, D, 1, false>);
    }
}

const void *split_kernel_ptr(int kv, int d, int gw, bool mfma) {
    if (kv == DA_F32) return d == 64 ? split_kernel_ptr<DA_F32, 64>(gw, false) : split_kernel_ptr<DA_F32, 128>(gw, false);
    if (kv == DA_BF16) return d == 64 ? split_kernel_ptr<DA_BF16, 64>(gw, mfma) : split_kernel_ptr<DA_BF16, 128>(gw, mfma);
    if (kv == DA_INT8) return d == 64 ? split_kernel_ptr<DA_INT8, 64>(gw, mfma) : split_kernel_ptr<DA_INT8, 128>(gw, mfma);
    return d == 64 ? split_kernel_ptr<DA_FP8_E4M3FN, 64>(gw, mfma) : split_kernel_ptr<DA_FP8_E4M3FN, 128>(gw, mfma);
}

// single_ok: the caller is a one-call entry point (decode_attn_run, decode_attn_append_run,
// decode_attn_run_static), which may take the single pass.
int make_plan(const da_desc *d, int max_len, Plan *p, bool single_ok = false) {
    int rc = validate(d);
    if (rc) return rc;
    if (max_len < 1 || max_len > d->cap)
        return fail(DA_ERR_INVALID_ARG, "max_len (%d) must be in [1, cap = %d]", max_len, d->cap);
    // The kernels address one (sequence, KV head) slot through buffer resources whose size and
    // lane offsets are 32-bit: every row a pass may touch (up to max_len, plus the prefetches
    // that run past a segment's end, under kSlotSlack bytes) must lie below 4 GiB.
    const int64_t row_bytes = (int64_t)d->d_k * elem_size(d->kv_dtype);
    if ((int64_t)max_len * row_bytes > (int64_t)UINT32_MAX - kSlotSlack)
        return fail(DA_ERR_UNSUPPORTED, "max_len %d rows of %lld bytes exceed the 4 GiB a (sequence, KV head) slot may span",
                    max_len, (long long)row_bytes);
    rc = plan_tiles(d, p);
    if (rc) return rc;
    const int64_t units = (int64_t)d->batch * d->h_kv * p->tiles;
    const int64_t rows_max = units * max_len;  // rows of all units at max_len
    int64_t nwg;
    if (d->block_rows) {
        nwg = (rows_max + d->block_rows - 1) / d->block_rows;
    } else {
        const bool ring32 = p->mfma && p->gw == 32 && d->kv_dtype == DA_BF16;
        nwg = resident_workgroups(split_kernel_ptr(d->kv_dtype, d->d_k, p->gw, p->mfma), ring32 ? 1 : kBlocksPerCu);
        // Vector ALUs with exactly one unit per CU (MHA, 8 x 32 heads on 256 CUs): one workgroup
        // per unit, so that at full length every unit is one segment written straight to out and
        // the combine has nothing to merge (MHA step 86.3 -> 84.6 us; on the 8-bit matrix-core
        // stages the same count was slower for int8 and no faster for fp8).
        if (!p->mfma && units == cu_count() && nwg > units) nwg = units;
        nwg = std::min<int64_t>(nwg, (rows_max + kMinRowsPerBlock - 1) / kMinRowsPerBlock);
    }
    p->nwg = (int)std::max<int64_t>(1, std::min<int64_t>(nwg, 1 << 20));
    // the single pass's tiling (vector ALUs) and splits per unit; it fails only for the
    // matrix-core flavour, which the single pass does not have
    Plan v = *p;
    const int rc_single = plan_tiles(d, &v, true);
    const int64_t units_single = rc_single ? 0 : (int64_t)d->batch * d->h_kv * v.tiles;
    p->nsplit = (int)std::min<int64_t>(kMaxSingleSplits, std::max<int64_t>(1, (max_len + kSingleRows - 1) / kSingleRows));
    // workspace: the partial rows of either path, and the single pass's counters (which the
    // split path never writes, so that they stay at zero)
    const size_t part_rows = std::max<size_t>(((size_t)p->nwg + units) * p->gt,
                                              (size_t)units_single * p->nsplit * (rc_single ? 0 : v.gt));
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    p->lens_off = kHeaderBytes;
    p->cnt_off = p->lens_off + up((size_t)d->batch * sizeof(int32_t));
    p->ncnt = (size_t)(d->batch + units_single);
    p->unit_off = p->cnt_off + up((size_t)(d->batch + units_single) * sizeof(int32_t));
    p->ml_off = p->unit_off + up((size_t)units * sizeof(int2));
    p->o_off = p->ml_off + up(part_rows * 2 * sizeof(float));
    p->bytes = p->o_off + up(part_rows * d->d_v * sizeof(float));
    p->single = false;
    if (single_ok && d->path != DA_PATH_SPLIT && d->block_rows == 0) {
        if (rc_single && d->path == DA_PATH_SINGLE) return rc_single;
        const int64_t seq_bytes = (int64_t)d->h_kv * v.tiles * max_len * 2 * row_bytes;
        if (!rc_single && (d->path == DA_PATH_SINGLE || seq_bytes <= kSingleMaxBytes)) {
            p->single = true;
            p->mfma = false;
            p->gt = v.gt;
            p->gw = v.gw;
            p->tiles = v.tiles;
        }
    }
    return DA_OK;
}

int launch_status(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return DA_OK;
}

template <int KV, int D, bool DIRECT>
void launch_split_gt(int gw, dim3 grid, hipStream_t st, const SplitArgs &args) {
    if constexpr (KV == DA_F32) {
        if (gw == 8) {
            hipLaunchKernelGGL((split_kv_attn_kernel<KV, D, 8, DIRECT>), grid, dim3(kBlock), 0, st, args);
            return;
        }
    }
    switch (gw) {
    case 4: hipLaunchKernelGGL((split_kv_attn_kernel<KV, D, 4, DIRECT>), grid, dim3(kBlock), 0, st, args); break;
    case 2: hipLaunchKernelGGL((split_kv_attn_kernel<KV, D, 2, DIRECT>), grid, dim3(kBlock), 0, st, args); break;
    default: hipLaunchKernelGGL((split_kv_attn_kernel<KV, D, 1, DIRECT>), grid, dim3(kBlock), 0, st, args); break;
    }
}

template <int KV, int D, bool DIRECT>
void launch_split_mfma_gt(int gw, dim3 grid, hipStream_t st, const SplitArgs &args) {
    if (gw == 32)
        hipLaunchKernelGGL((split_kv_attn_mfma_kernel<KV, D, 32, DIRECT>), grid, dim3(kBlock), 0, st, args);
    else
        hipLaunchKernelGGL((split_kv_attn_mfma_kernel<KV, D, 16, DIRECT>), grid, dim3(kBlock), 0, st, args);
}

template <bool DIRECT>
void launch_split(int kv, int d, int gw, bool mfma, dim3 grid, hipStream_t st, const SplitArgs &args) {
    if (mfma) {
        if (kv == DA_BF16) {
            if (d == 64) launch_split_mfma_gt<DA_BF16, 64, DIRECT>(gw, grid, st, args);
            else launch_split_mfma_gt<DA_BF16, 128, DIRECT>(gw, grid, st, args);
        } else if (kv == DA_INT8) {
            if (d == 64) launch_split_mfma_gt<DA_INT8, 64, DIRECT>(gw, grid, st, args);
            else launch_split_mfma_gt<DA_INT8, 128, DIRECT>(gw, grid, st, args);
        } else {
            if (d == 64) launch_split_mfma_gt<DA_FP8_E4M3FN, 64, DIRECT>(gw, grid, st, args);
            else launch_split_mfma_gt<DA_FP8_E4M3FN, 128, DIRECT>(gw, grid, st, args);
        }
        return;
    }
    if (kv == DA_F32) {
        if (d == 64) launch_split_gt<DA_F32, 64, DIRECT>(gw, grid, st, args);
        else launch_split_gt<DA_F32, 128, DIRECT>(gw, grid, st, args);
    } else if (kv == DA_BF16) {
        if (d == 64) launch_split_gt<DA_BF16, 64, DIRECT>(gw, grid, st, args);
        else launch_split_gt<DA_BF16, 128, DIRECT>(gw, grid, st, args);
    } else if (kv == DA_INT8) {
        if (d == 64) launch_split_gt<DA_INT8, 64, DIRECT>(gw, grid, st, args);
        else launch_split_gt<DA_INT8, 128, DIRECT>(gw, grid, st, args);
    } else {
        if (d == 64) launch_split_gt<DA_FP8_E4M3FN, 64, DIRECT>(gw, grid, st, args);
        else launch_split_gt<DA_FP8_E4M3FN, 128, DIRECT>(gw, grid, st, args);
    }
}

template <int KV, int D>
void launch_single_gw(int gw, dim3 grid, hipStream_t st, const SplitArgs &args) {
    if constexpr (KV == DA_F32) {
        if (gw == 8) {
            hipLaunchKernelGGL((decode_step_single_kernel<KV, D, 8>), grid, dim3(kBlock), 0, st, args);
            return;
        }
    }
    switch (gw) {
    case 4: hipLaunchKernelGGL((decode_step_single_kernel<KV, D, 4>), grid, dim3(kBlock), 0, st, args); break;
    case 2: hipLaunchKernelGGL((decode_step_single_kernel<KV, D, 2>), grid, dim3(kBlock), 0, st, args); break;
    default: hipLaunchKernelGGL((decode_step_single_kernel<KV, D, 1>), grid, dim3(kBlock), 0, st, args); break;
    }
}

void launch_single(int kv, int d, int gw, dim3 grid, hipStream_t st, const SplitArgs &args) {
    if (kv == DA_F32) {
        if (d == 64) launch_single_gw<DA_F32, 64>(gw, grid, st, args);
        else launch_single_gw<DA_F32, 128>(gw, grid, st, args);
    } else if (kv == DA_BF16) {
        if (d == 64) launch_single_gw<DA_BF16, 64>(gw, grid, st, args);
        else launch_single_gw<DA_BF16, 128>(gw, grid, st, args);
    } else if (kv == DA_INT8) {
        if (d == 64) launch_single_gw<DA_INT8, 64>(gw, grid, st, args);
        else launch_single_gw<DA_INT8, 128>(gw, grid, st, args);
    } else {
        if (d == 64) launch_single_gw<DA_FP8_E4M3FN, 64>(gw, grid, st, args);
        else launch_single_gw<DA_FP8_E4M3FN, 128>(gw, grid, st, args);
    }
}

Partition partition_of(const da_desc *desc, const Plan &p, int max_len, bool append) {
    Partition pt;
    pt.batch = desc->batch;
    pt.h_kv = desc->h_kv;
    pt.tiles = p.tiles;
    pt.max_len = max_len;
    pt.nwg = p.nwg;
    pt.append_cap = append ? desc->cap : 0;
    pt.nq = n_queries(desc);
    return pt;
}

// Checks the run arguments and launches the split kernel: with out non-NULL (the one-call entry
// points), units that one workgroup covers are written to out directly, or the plan may take
// the single pass, which writes every output itself (*whole = true: no combine follows);
// otherwise every segment writes its partial result (decode_attn_partial). Device error bits go
// to err_word when it is given, else to the workspace's own error word.
int run_split(const da_desc *desc, const void *q, const void *k_cache, const void *v_cache, const int32_t *lens,
              const void *k_new, const void *v_new, int32_t max_len, const float *kv_scales, float *out,
              void *workspace, size_t ws_bytes, void *stream, const char *who, int32_t *err_word = nullptr,
              bool *whole = nullptr, int32_t *counters = nullptr, size_t max_counters = 0) {
    Plan p;
    int rc = make_plan(desc, max_len, &p, out != nullptr);
    if (rc) return rc;
    if (p.single && counters && p.ncnt > max_counters) {  // too many counters for the caller's area
        if (desc->path == DA_PATH_SINGLE)
            return fail(DA_ERR_UNSUPPORTED, "%s: the single pass needs %zu counters, %zu available", who, p.ncnt,
                        max_counters);
        da_desc split = *desc;
        split.path = DA_PATH_SPLIT;
        rc = make_plan(&split, max_len, &p, true);
        if (rc) return rc;
    }
    if (whole) *whole = p.single;
    if (!q || !k_cache || !v_cache || !lens || !workspace)
        return fail(DA_ERR_INVALID_ARG, "%s: a buffer pointer is NULL", who);
    const bool append = k_new || v_new;
    if (append && n_queries(desc) > 1)
        return fail(DA_ERR_UNSUPPORTED, "%s: the fused append takes one query per sequence (n_queries %d)", who,
                    desc->n_queries);
    if (append && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)))
        return fail(DA_ERR_INVALID_ARG, "%s: k_new and v_new must both be 16-byte aligned device pointers", who);
    if ((desc->kv_dtype == DA_FP8_E4M3FN || desc->kv_dtype == DA_INT8) && !kv_scales)
        return fail(DA_ERR_INVALID_ARG, "%s: an 8-bit (fp8 / int8) cache needs kv_scales", who);
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
    args.lens = const_cast<int32_t *>(lens);  // written by the single pass with an append only
    args.kv_scales = kv_scales;
    args.part_ml = reinterpret_cast<float *>(ws + p.ml_off);
    args.part_o = reinterpret_cast<float *>(ws + p.o_off);
    args.out = out;
    args.h_q = desc->h_q;
    args.cap = desc->cap;
    args.pt = partition_of(desc, p, max_len, append);
    args.qk_scale = desc->scale * kLog2e;
    args.k_new = k_new;
    args.v_new = v_new;
    args.lens_copy = reinterpret_cast<int32_t *>(ws + p.lens_off);
    args.err = err_word ? err_word : reinterpret_cast<int32_t *>(ws);
    args.row_bytes = desc->d_k * elem_size(desc->kv_dtype);
    args.shared_lines = args.row_bytes % kCacheLine != 0 || reinterpret_cast<uintptr_t>(k_cache) % kCacheLine != 0 ||
                        reinterpret_cast<uintptr_t>(v_cache) % kCacheLine != 0;
    args.unit_wg = reinterpret_cast<int2 *>(ws + p.unit_off);
    args.dv = desc->d_v;
    args.gt = p.gt;
    args.grp_rows = group_rows(desc);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.single) {
        args.nsplit = p.nsplit;
        args.seq_cnt = counters ? counters : reinterpret_cast<int32_t *>(ws + p.cnt_off);
        args.unit_cnt = args.seq_cnt + desc->batch;
        const int64_t grid = (int64_t)desc->batch * desc->h_kv * p.tiles * p.nsplit;
        launch_single(desc->kv_dtype, desc->d_k, p.gw, dim3((unsigned)grid), st, args);
        return launch_status("decode_step_single_kernel");
    }
    if (out)
        launch_split<true>(desc->kv_dtype, desc->d_k, p.gw, p.mfma, dim3(p.nwg), st, args);
    else
        launch_split<false>(desc->kv_dtype, desc->d_k, p.gw, p.mfma, dim3(p.nwg), st, args);
    return launch_status("split_kv_attn_kernel");
}

int run_combine(const da_desc *desc, int32_t *lens, int32_t max_len, float *out, void *workspace,
                size_t ws_bytes, void *stream, int skip_single, bool append, const char *who,
                int32_t *err_word = nullptr, float *lse = nullptr) {
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
    const int2 *uw = reinterpret_cast<const int2 *>(ws + p.unit_off);
    const float *po = reinterpret_cast<const float *>(ws + p.o_off);
    int32_t *err = err_word ? err_word : reinterpret_cast<int32_t *>(ws);
    if (append && n_queries(desc) > 1)
        return fail(DA_ERR_UNSUPPORTED, "%s: the fused append takes one query per sequence (n_queries %d)", who,
                    desc->n_queries);
    // rows of a unit per workgroup: more rows per workgroup spread the fixed cost (the length,
    // the unit's entry, the merge) over more rows while at least two workgroups per CU remain
    // and each segment group keeps at most one load batch (a unit has about nwg / units + 1
    // segments); with 2048 rows over 256 CUs, 4 rows per workgroup took the combine from 6.5
    // to 4.5 us, while fewer than two workgroups per CU were slower
    // Too few rows for that (a few units of many segments): column slices instead, down to half
    // a row (16 threads per segment group for d = 128). On MQA (128 rows of 64 segments) halves
    // took the combine from 6.3 to 4.9 us; quarters (5.3) and eighths (7.1) were slower.
    const int64_t units = (int64_t)desc->batch * desc->h_kv * p.tiles;
    const int groups = kCombineBlock / (desc->d_v / 4);  // segment groups of a workgroup
    const int64_t segs = p.nwg / units + 1;
    const int64_t min_wg = 2 * (int64_t)cu_count();
    int rw = 1, cs = 1;
    while (2 * rw <= groups && p.gt % (2 * rw) == 0 && 2 * rw * segs <= 8 * groups &&
           units * (p.gt / (2 * rw)) >= min_wg)
        rw *= 2;
    while (rw == 1 && 2 * cs <= 2 && units * p.gt * cs < min_wg) cs *= 2;
    const dim3 grid((unsigned)(units * (p.gt / rw) * cs));
    const Partition pt = partition_of(desc, p, max_len, append);
    // appending: stored lengths from the split kernel's copy, new lengths written to lens
    const int32_t *lsrc = append ? reinterpret_cast<const int32_t *>(ws + p.lens_off) : lens;
    int32_t *lupd = append ? lens : nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (desc->d_v == 64)
        hipLaunchKernelGGL(lse_combine_kernel<64>, grid, dim3(kCombineBlock), 0, st, lsrc, lupd, uw, ml, po, out, err,
                           desc->h_q, p.gt, group_rows(desc), rw, cs, pt, skip_single, lse);
    else
        hipLaunchKernelGGL(lse_combine_kernel<128>, grid, dim3(kCombineBlock), 0, st, lsrc, lupd, uw, ml, po, out, err,
                           desc->h_q, p.gt, group_rows(desc), rw, cs, pt, skip_single, lse);
    return launch_status("lse_combine_kernel");
}

// Scratch of decode_attn_run_static: the workspace of decode_attn_run for callers that cannot
// allocate. One copy per device, held from the library's load on that device until the process
// ends. Host code never uses the array's name as an address (on the host it is only a stand-in
// for the symbol): the device address comes from hipGetSymbolAddress, once per device.
// Its first kStaticCounterBytes hold the single pass's arrival counters, which start at zero
// (static storage) and which every single pass leaves at zero; no other use of the scratch
// writes them, whatever the descriptor. The plan's workspace follows.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
constexpr size_t kStaticCounterBytes = size_t(256) << 10;
__device__ __align__(256) char scratch[kStaticScratchBytes];

// Device address of this device's scratch (looked up on the first call on each device).
int static_scratch(void **ptr) {
    static std::mutex mu;
    static std::map<int, void *> addr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DA_ERR_LAUNCH, "decode_attn_run_static: hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(mu);
    auto it = addr.find(dev);
    if (it == addr.end()) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(DA_ERR_LAUNCH, "decode_attn_run_static: scratch address on device %d: %s", dev,
                        hipGetErrorString(e));
        it = addr.emplace(dev, p).first;
    }
    *ptr = it->second;
    return DA_OK;
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

int da_plan(const da_desc *desc, int32_t max_len, int32_t *rows_per_block, int32_t *n_blocks,
            int32_t *heads_per_block_out, int32_t *path_out) {
    Plan p;
    const int rc = make_plan(desc, max_len, &p, true);
    if (rc) return rc;
    const int64_t rows_max = (int64_t)desc->batch * desc->h_kv * p.tiles * max_len;
    const int64_t nwg = p.single ? (int64_t)desc->batch * desc->h_kv * p.tiles * p.nsplit : p.nwg;
    if (rows_per_block) *rows_per_block = (int32_t)((rows_max + nwg - 1) / nwg);
    if (n_blocks) *n_blocks = (int32_t)nwg;
    if (heads_per_block_out) *heads_per_block_out = p.gt;
    if (path_out) *path_out = p.single ? DA_PATH_SINGLE : DA_PATH_SPLIT;
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
    return run_split(desc, q, k_cache, v_cache, lens, nullptr, nullptr, max_len, kv_scales, nullptr, workspace,
                     ws_bytes, stream, "decode_attn_partial");
}

int decode_attn_combine(const da_desc *desc, const int32_t *lens, int32_t max_len, float *out, void *workspace,
                        size_t ws_bytes, void *stream) {
    return run_combine(desc, const_cast<int32_t *>(lens), max_len, out, workspace, ws_bytes, stream, 0, false,
                       "decode_attn_combine");
}

int decode_attn_run(const da_desc *desc, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *lens, int32_t max_len, const float *kv_scales, float *out, void *workspace,
                    size_t ws_bytes, void *stream) {
    if (!out) return fail(DA_ERR_INVALID_ARG, "decode_attn_run: out is NULL");
    bool whole = false;
    const int rc = run_split(desc, q, k_cache, v_cache, lens, nullptr, nullptr, max_len, kv_scales, out, workspace,
                             ws_bytes, stream, "decode_attn_run", nullptr, &whole);
    if (rc || whole) return rc;
    return run_combine(desc, const_cast<int32_t *>(lens), max_len, out, workspace, ws_bytes, stream, 1, false,
                       "decode_attn_run");
}

int decode_attn_append_partial(const da_desc *desc, const void *q, void *k_cache, void *v_cache,
                               const int32_t *lens, const void *k_new, const void *v_new, int32_t max_len,
                               const float *kv_scales, void *workspace, size_t ws_bytes, void *stream) {
    if (!k_new || !v_new) return fail(DA_ERR_INVALID_ARG, "decode_attn_append_partial: k_new or v_new is NULL");
    return run_split(desc, q, k_cache, v_cache, lens, k_new, v_new, max_len, kv_scales, nullptr, workspace,
                     ws_bytes, stream, "decode_attn_append_partial");
}

int decode_attn_append_combine(const da_desc *desc, int32_t *lens, int32_t max_len, float *out, void *workspace,
                               size_t ws_bytes, void *stream) {
    return run_combine(desc, lens, max_len, out, workspace, ws_bytes, stream, 0, true,
                       "decode_attn_append_combine");
}

int decode_attn_append_run(const da_desc *desc, const void *q, void *k_cache, void *v_cache, int32_t *lens,
                           const void *k_new, const void *v_new, int32_t max_len, const float *kv_scales,
                           float *out, void *workspace, size_t ws_bytes, void *stream) {
    if (!out) return fail(DA_ERR_INVALID_ARG, "decode_attn_append_run: out is NULL");
    if (!k_new || !v_new) return fail(DA_ERR_INVALID_ARG, "decode_attn_append_run: k_new or v_new is NULL");
    bool whole = false;
    const int rc = run_split(desc, q, k_cache, v_cache, lens, k_new, v_new, max_len, kv_scales, out, workspace,
                             ws_bytes, stream, "decode_attn_append_run", nullptr, &whole);
    if (rc || whole) return rc;
    return run_combine(desc, lens, max_len, out, workspace, ws_bytes, stream, 1, true, "decode_attn_append_run");
}

int decode_attn_run_static(const da_desc *desc, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *lens, int32_t max_len, const float *kv_scales, float *out,
                           int32_t *dev_err, void *stream) {
    if (!out) return fail(DA_ERR_INVALID_ARG, "decode_attn_run_static: out is NULL");
    if (dev_err && (reinterpret_cast<uintptr_t>(dev_err) & 3u))
        return fail(DA_ERR_INVALID_ARG, "decode_attn_run_static: dev_err is not 4-byte aligned");
    Plan p;
    int rc = make_plan(desc, max_len, &p);
    if (rc) return rc;
    if (p.bytes > kStaticScratchBytes - kStaticCounterBytes)
        return fail(DA_ERR_WORKSPACE, "decode_attn_run_static: needs %zu bytes of scratch, the static scratch holds %zu",
                    p.bytes, kStaticScratchBytes - kStaticCounterBytes);
    void *base = nullptr;
    rc = static_scratch(&base);
    if (rc) return rc;
    int32_t *counters = static_cast<int32_t *>(base);
    void *ws = static_cast<char *>(base) + kStaticCounterBytes;
    // without dev_err the error bits land in the scratch's own error word, which nothing reads
    int32_t *err = dev_err ? dev_err : static_cast<int32_t *>(ws);
    bool whole = false;
    rc = run_split(desc, q, k_cache, v_cache, lens, nullptr, nullptr, max_len, kv_scales, out, ws, p.bytes, stream,
                   "decode_attn_run_static", err, &whole, counters, kStaticCounterBytes / sizeof(int32_t));
    if (rc || whole) return rc;
    return run_combine(desc, const_cast<int32_t *>(lens), max_len, out, ws, p.bytes, stream, 1, false,
                       "decode_attn_run_static", err);
}

int decode_attn_run_lse(const da_desc *desc, const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *lens, int32_t max_len, const float *kv_scales, float *out, float *lse,
                        void *workspace, size_t ws_bytes, void *stream) {
    if (!out || !lse) return fail(DA_ERR_INVALID_ARG, "decode_attn_run_lse: out and lse must not be NULL");
    if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(DA_ERR_INVALID_ARG, "decode_attn_run_lse: lse is not 4-byte aligned");
    // every unit leaves partials (no direct writes, no single pass): the combine writes out and lse
    const int rc = run_split(desc, q, k_cache, v_cache, lens, nullptr, nullptr, max_len, kv_scales, nullptr,
                             workspace, ws_bytes, stream, "decode_attn_run_lse");
    if (rc) return rc;
    return run_combine(desc, const_cast<int32_t *>(lens), max_len, out, workspace, ws_bytes, stream, 0, false,
                       "decode_attn_run_lse", nullptr, lse);
}

int decode_attn_merge_lse(int64_t rows, int32_t d, int32_t shards, const float *outs, const float *lses, float *out,
                          float *lse, void *stream) {
    if (rows < 0 || d < 4 || d % 4 || d > 4096 || shards < 1 || shards > 4096)
        return fail(DA_ERR_INVALID_ARG, "decode_attn_merge_lse: rows %lld, d %d (a positive multiple of 4, at most 4096), "
                                        "shards %d (1..4096)", (long long)rows, d, shards);
    if (rows == 0) return DA_OK;
    if (!outs || !lses || !out) return fail(DA_ERR_INVALID_ARG, "decode_attn_merge_lse: a buffer pointer is NULL");
    if (!aligned16(outs) || !aligned16(out) || (reinterpret_cast<uintptr_t>(lses) & 3u) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return fail(DA_ERR_INVALID_ARG, "decode_attn_merge_lse: outs and out must be 16-byte aligned, lses and lse 4-byte");
    const int64_t threads = rows * (d / 4);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return fail(DA_ERR_INVALID_ARG, "decode_attn_merge_lse: too many rows");
    hipLaunchKernelGGL(merge_lse_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), rows, d,
                       shards, outs, lses, out, lse);
    return launch_status("merge_lse_kernel");
}

int da_stream_read(const void *buf, size_t bytes, float *sink, void *stream) {
    if (!buf || !sink) return fail(DA_ERR_INVALID_ARG, "da_stream_read: NULL pointer");
    if (!aligned16(buf) || bytes % 16 || bytes == 0)
        return fail(DA_ERR_INVALID_ARG, "da_stream_read: buf must be 16-byte aligned and bytes a positive multiple of 16");
    const size_t step = 256u * 16u * kStreamUnroll;
    const size_t chunk = (bytes / kStreamWorkgroups + step - 1) / step * step;
    if (chunk > 0x7FFFFFFFull) return fail(DA_ERR_INVALID_ARG, "da_stream_read: more than 1 TiB");
    hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamWorkgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const char *>(buf), bytes, (uint32_t)chunk, sink);
    return launch_status("da_stream_read");
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
