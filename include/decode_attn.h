/*
 * decode_attn.h -- C ABI of the MI355X (gfx950) split-KV decode-attention library.
 *
 * The operation (page "MoA-Structured Decode Attention", §2 Decode DNF, eqs. (1)-(3)):
 * for every sequence b and query head h, with n = lens[b] cached rows,
 *     s[l]   = scale * sum_j q[b,h,j] * K[b,kvh,l,j]            (Step I, K read row by row)
 *     a      = softmax(s)  (max subtracted, exponentials normalised)   (Step II)
 *     out[d] = sum_l a[l] * V[b,kvh,l,d]                          (Step III)
 * where kvh = h / (h_q / h_kv) selects the query head's KV group (same page, §6 GQA/MQA:
 * the group is selected, never broadcast-copied), and one row per step is appended to the
 * cache at its row-major offset (same page, §5 KV-cache accumulation).
 *
 * Layouts (all row-major, contiguous; the same page's §4 gamma offsets lifted to rank 4):
 *   q        [batch, h_q, d_k]          element type desc->q_dtype ([batch, T, h_q, d_k] for
 *                                       T = desc->n_queries > 1 query rows per sequence)
 *   k_cache  [batch, h_kv, cap, d_k]    element type desc->kv_dtype;
 *                                       element (b,kvh,l,j) at ((b*h_kv+kvh)*cap+l)*d_k+j
 *   v_cache  [batch, h_kv, cap, d_v]    element type desc->kv_dtype
 *   lens     [batch] int32              rows currently in each sequence (device memory)
 *   kv_scales[batch, h_kv, 2] fp32      (K scale, V scale) per slot; 8-bit caches only
 *   out      [batch, h_q, d_v] fp32     ([batch, T, h_q, d_v] for T > 1)
 * For an fp8 cache the value of an element is decode_e4m3fn(code) * its slot's scale; for
 * an int8 cache it is the two's-complement code * its slot's scale (the decode-attention
 * roofline page: 8-bit KV, fp8 or int8, halves the bytes each step reads).
 *
 * Memory and threads: the caller owns every buffer (all pointers are device pointers unless
 * stated otherwise). The library never allocates or frees device memory and keeps no
 * pointers between calls. Every launch is asynchronous on the caller's stream (a
 * hipStream_t passed as void*; NULL means the default stream); nothing on the run path
 * synchronises the host. Calls are thread-safe.
 *
 * Errors: every function returns DA_OK (0) or a negative DA_ERR_* code, checked on the host
 * before anything is launched; on failure nothing is launched. da_last_error() gives a
 * per-thread message for the latest failure. Conditions only the device can see (a lens
 * value out of range) cannot be returned without a synchronisation: the kernel then skips
 * the affected work, writes zeros where it would have written results, and ORs a
 * DA_DEV_ERR_* bit into the workspace's sticky error word, which da_read_device_error reads.
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host-side status codes. */
#define DA_OK 0
#define DA_ERR_INVALID_ARG (-1) /* null or misaligned pointer, bad shape, h_q % h_kv != 0,
                                   max_len outside [1, cap], non-finite scale */
#define DA_ERR_UNSUPPORTED (-2) /* head size or dtype combination not built, a slot of 4 GiB
                                   or more, the matrix-core flavour asked for an fp32 cache */
#define DA_ERR_WORKSPACE (-3)   /* workspace smaller than da_workspace_size() */
#define DA_ERR_LAUNCH (-4)      /* the HIP runtime refused a launch (see da_last_error) */

/* Device-side error bits, ORed into the workspace's error word. */
#define DA_DEV_ERR_APPEND_FULL 1 /* kv_append: lens[b] outside [0, cap); row b not written,
                                    lens[b] unchanged */
#define DA_DEV_ERR_LEN_RANGE 2   /* decode: lens[b] outside [max(1, n_queries), max_len]; out[b] zeroed */

typedef enum { DA_F32 = 0, DA_BF16 = 1, DA_FP8_E4M3FN = 2, DA_INT8 = 3 } da_dtype;

/* Kernel flavour (da_desc.flavour): the library's choice, or one flavour asked for (to measure
 * both on one shape). The matrix-core flavour takes bf16, fp8 and int8 caches only. */
typedef enum { DA_FLAVOUR_AUTO = 0, DA_FLAVOUR_VECTOR = 1, DA_FLAVOUR_MATRIX = 2 } da_flavour;

/* Launch path of the one-call entry points (da_desc.path): the library's choice; the split
 * path (split kernel + log-sum-exp combine, two launches); or the single pass (one launch). */
typedef enum { DA_PATH_AUTO = 0, DA_PATH_SPLIT = 1, DA_PATH_SINGLE = 2 } da_path;

/*
 * Problem descriptor. Supported: d_k == d_v in {64, 128}; (q_dtype, kv_dtype) in
 * {(F32, F32), (BF16, BF16), (BF16, FP8_E4M3FN), (BF16, INT8)}; any h_q that is a
 * multiple of h_kv; batch <= 1024. scale is the factor of Step I (1/sqrt(d_k) in the page's
 * setting), applied once. Work partition: the cache rows of all (sequence, KV head) pairs,
 * taken in order, are cut into equal contiguous shares, one per workgroup. block_rows = 0
 * lets the library use one share per workgroup that fits on the device at once;
 * block_rows > 0 asks for shares of about block_rows rows at max_len instead.
 *
 * n_queries (T; 0 or 1: single-query decode, at most 1024) is the number of query rows per
 * sequence, for speculative decoding or a chunked prefill: q and out are then
 * [batch, T, h_q, d], and query t of sequence b, at position lens[b] - T + t, attends over
 * rows [0, lens[b] - T + 1 + t) of the cache (causal: its own row and every earlier one; the
 * T newest rows are the queries' own keys, already in the cache). Page "MoA-Structured Decode
 * Attention", introduction (the decode form is the forward form with the query-row index
 * fixed to the current step; here it spans the last T steps) and page "Phase 3, Section 6:
 * StoryLM-0 head-parallel attention", §3 (softmax over the key axis of the scaled scores
 * plus a mask, T query rows). lens[b] must be at least T (else the device error
 * DA_DEV_ERR_LEN_RANGE). The fused-append entry points take T = 1 only.
 *
 * Reads per KV row (same page, §6: the g query heads of a group select one copy of its rows):
 * the g * T query rows of a KV group share each K and V row read, once per head tile. With a
 * bf16, fp8 or int8 cache and g * T >= 3 (matrix cores) a tile holds up to 32 query rows, so
 * every group with g * T <= 32 reads its rows once (ceil(g * T / 32) times beyond); g * T <= 2
 * reads once on the vector ALUs; an fp32 cache reads once for g * T <= 8 (ceil(g * T / 8)
 * times beyond). da_plan's heads_per_block is the tile's query-row count.
 *
 * flavour (da_flavour): DA_FLAVOUR_AUTO (0) for the rule above; DA_FLAVOUR_VECTOR or
 * DA_FLAVOUR_MATRIX to run one flavour regardless (the vector ALUs then cut 8-bit and bf16
 * groups into tiles of up to 4 rows). Results agree within the tolerances either way.
 *
 * path (da_path) applies to the one-call entry points (decode_attn_run, decode_attn_append_run,
 * decode_attn_run_static); the two-stage entry points always take the split path. The single
 * pass runs the whole step in one kernel launch, on the vector ALUs: every (sequence, KV head,
 * head tile) is cut into ceil(max_len / 64) splits (at most 64) of one workgroup each; the
 * workgroup holding a sequence's new last row appends it first, each split leaves a partial
 * result in the workspace, and the split that finishes last merges the unit's partials into
 * out (no workgroup waits for another). It is for latency-bound problems, where a second
 * launch costs more than the rows. DA_PATH_AUTO (0) takes it when every sequence's K and V
 * bytes at max_len (over all its head tiles) are at most 1 MiB, and block_rows is 0;
 * DA_PATH_SINGLE asks for it whatever the size (block_rows must then be 0; it refuses
 * DA_FLAVOUR_MATRIX); DA_PATH_SPLIT never takes it. The single pass keeps arrival counters in
 * the workspace that rest at zero between calls: the workspace must have been zeroed by
 * da_workspace_init once, and again before it serves a descriptor with another batch, h_kv,
 * h_q, n_queries or head size (the static scratch of decode_attn_run_static needs nothing).
 */
typedef struct {
    int32_t batch;
    int32_t h_q;
    int32_t h_kv;
    int32_t d_k;
    int32_t d_v;
    int32_t cap;
    int32_t q_dtype;  /* da_dtype */
    int32_t kv_dtype; /* da_dtype */
    float scale;
    int32_t block_rows;
    int32_t n_queries; /* query rows per sequence; 0 or 1 = single-query decode */
    int32_t flavour;   /* da_flavour; 0 = the library's choice */
    int32_t path;      /* da_path; 0 = the library's choice */
} da_desc;

/*
 * Bytes of device workspace decode_attn_run / kv_append need for this descriptor when no
 * sequence is longer than max_len (1 <= max_len <= cap). The workspace holds the sticky
 * error word and the per-split partial results (running max, sum of exponentials and
 * unnormalised output of each split; see decode_attn_partial), with the bookkeeping the
 * combine needs to find them (the total row count and, per (sequence, KV head, head tile),
 * the first and last workgroup holding its rows). *bytes is written on the
 * host. A workspace serves one call at a time: calls that overlap on the same workspace race.
 */
int da_workspace_size(const da_desc *desc, int32_t max_len, size_t *bytes);

/*
 * Chosen work partition of the one-call entry points for (desc, max_len), all outputs host
 * int32 (any may be NULL): cache rows per workgroup when every sequence has max_len rows,
 * workgroups launched (for the single pass: batch * h_kv * head tiles * splits), query rows
 * per head tile, and the path taken (DA_PATH_SPLIT or DA_PATH_SINGLE).
 */
int da_plan(const da_desc *desc, int32_t max_len, int32_t *rows_per_block, int32_t *n_blocks,
            int32_t *heads_per_block, int32_t *path);

/*
 * Zeroes the whole workspace with a kernel (not a memset), clearing its error word. Call
 * once after allocating it, and before the workspace serves another descriptor (its single
 * pass counters must be at zero; every call leaves them so for its own descriptor).
 */
int da_workspace_init(void *workspace, size_t ws_bytes, void *stream);

/*
 * KV-cache accumulation (page "MoA-Structured Decode Attention", §5): for every sequence b
 * and KV head kvh, copies row k_new[b,kvh,:] (shape [batch, h_kv, d_k], kv_dtype) into row
 * lens[b] of k_cache and v_new[b,kvh,:] into row lens[b] of v_cache, then sets
 * lens[b] += 1. Bit copies: every other byte of the caches is unchanged. 8-bit rows
 * must already be quantised with their slot's scale. A sequence with lens[b] outside [0, cap) is
 * skipped and raises DA_DEV_ERR_APPEND_FULL in the workspace (which may be NULL when the
 * caller does not want the error word; the row is still skipped).
 */
int kv_append(const da_desc *desc, void *k_cache, void *v_cache, int32_t *lens,
              const void *k_new, const void *v_new, void *workspace, void *stream);

/*
 * Decode attention for every (b, h) over rows [0, lens[b]) (page "MoA-Structured Decode
 * Attention", §2 Steps I-III, §6 group selection). max_len is a host-side upper bound on
 * every lens[b] (1 <= max_len <= cap) that sizes the work partition. kv_scales is required
 * for an fp8 or int8 cache and ignored otherwise. out is fp32 [batch, h_q, d_v]. Two
 * kernels: the split kernel (a (sequence, KV head) whose rows one workgroup covers is
 * written to out directly, the others leave per-segment partial results) and the
 * log-sum-exp combine of the rest. The result equals decode_attn_partial followed by decode_attn_combine.
 */
int decode_attn_run(const da_desc *desc, const void *q, const void *k_cache,
                    const void *v_cache, const int32_t *lens, int32_t max_len,
                    const float *kv_scales, float *out, void *workspace, size_t ws_bytes,
                    void *stream);

/*
 * First stage of decode_attn_run: each workgroup reads its share of K and V rows once for
 * all query heads of the group and writes, per (sequence, KV head) segment of its share and
 * per query head, the running max (base-2 exponent domain), the sum of exponentials and the
 * unnormalised output row to the workspace, and records which workgroups hold each
 * (sequence, KV head, head tile)'s rows.
 */
int decode_attn_partial(const da_desc *desc, const void *q, const void *k_cache,
                        const void *v_cache, const int32_t *lens, int32_t max_len,
                        const float *kv_scales, void *workspace, size_t ws_bytes, void *stream);

/*
 * Second stage: merges the segments of every (b, h) by their log-sum-exp weights into out
 * (an exact rewriting of Step II's normalisation over the whole row range).
 */
int decode_attn_combine(const da_desc *desc, const int32_t *lens, int32_t max_len, float *out,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * One decode step with the append fused into the attention pass (page "MoA-Structured Decode
 * Attention", §5 accumulation, then §2 Steps I-III): the same results, cache bytes, lengths
 * and error bits as kv_append(k_new, v_new) followed by decode_attn_run, in two kernels
 * instead of three. The split kernel attends over lens[b] + 1 rows (lens[b] rows for a
 * sequence whose append is skipped because lens[b] is outside [0, cap); that raises
 * DA_DEV_ERR_APPEND_FULL); each workgroup whose share ends at a sequence's new last row
 * stores that row into the cache before reading it. The combine kernel then sets
 * lens[b] += 1 for the appended sequences. max_len bounds the lengths after the append
 * (lens[b] + 1 <= max_len <= cap). k_cache, v_cache and lens are written; k_new and v_new
 * are [batch, h_kv, d] rows in the cache's type, 8-bit rows quantised with their slot's scale.
 * The workspace's error word must be the one the caller reads (it is not optional here).
 */
int decode_attn_append_run(const da_desc *desc, const void *q, void *k_cache, void *v_cache,
                           int32_t *lens, const void *k_new, const void *v_new, int32_t max_len,
                           const float *kv_scales, float *out, void *workspace, size_t ws_bytes,
                           void *stream);

/*
 * First stage of decode_attn_append_run: stores the new rows where the attention pass reads
 * them and writes the per-segment partial results, plus a copy of the stored lengths in the
 * workspace. lens is read, not changed: decode_attn_append_combine, on the same workspace and
 * stream, updates it.
 */
int decode_attn_append_partial(const da_desc *desc, const void *q, void *k_cache, void *v_cache,
                               const int32_t *lens, const void *k_new, const void *v_new,
                               int32_t max_len, const float *kv_scales, void *workspace,
                               size_t ws_bytes, void *stream);

/*
 * Second stage of decode_attn_append_run: merges every (b, h) into out using the lengths
 * copied by decode_attn_append_partial, then writes the new lengths to lens.
 */
int decode_attn_append_combine(const da_desc *desc, int32_t *lens, int32_t max_len, float *out,
                               void *workspace, size_t ws_bytes, void *stream);

/*
 * decode_attn_run without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops that must not allocate, harnesses that forbid
 * it). Same arguments, kernels and results as decode_attn_run (bit for bit), except:
 *   - the split partials live in a static scratch array the library holds on each device it
 *     runs on (16 MiB, kept until the process ends): 256 KiB of it for the single pass's
 *     counters, the rest for the workspace; a (desc, max_len) whose da_workspace_size()
 *     exceeds 16 MiB - 256 KiB is rejected with DA_ERR_WORKSPACE, nothing launched (and one
 *     whose single pass would need more than 65536 counters takes the split path);
 *   - dev_err (device int32, caller-owned, 4-byte aligned, may be NULL) receives the
 *     DA_DEV_ERR_* bits ORed in, as the workspace's error word does for decode_attn_run; the
 *     caller clears it. With NULL the bits are dropped (the work is still skipped and zeroed).
 * Nothing is allocated or freed on any call. Every call on a device shares that device's
 * scratch, which keeps the last call's contents (no part of it needs clearing between calls):
 * calls that overlap on one device (other streams, other threads) race and must be ordered
 * by the caller.
 */
int decode_attn_run_static(const da_desc *desc, const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *lens, int32_t max_len,
                           const float *kv_scales, float *out, int32_t *dev_err, void *stream);

/*
 * decode_attn_run over one shard of the rows, for a context split over several devices: each
 * device holds a contiguous part of every sequence's rows as a cache of its own (lens[b] rows
 * of it, 0 allowed) and emits, per query row, the attention over its part together with that
 * part's log-sum-exp; decode_attn_merge_lse then merges the parts into attention over all the
 * rows (page "MoA-Structured Decode Attention", §2 eq. (2): the softmax normalisation over a
 * union of row sets is the log-sum-exp-weighted combination of the normalisations over each
 * set). Arguments as decode_attn_run, plus
 *   lse  [batch, h_q] fp32 ([batch, T, h_q] for T = n_queries > 1), 4-byte aligned:
 *        ln sum_l exp(scale * q . K[l]) over the rows the query attends to (natural log).
 * A sequence with lens[b] = 0 holds no rows of this shard: its out rows are 0 and its lse
 * -inf, with no device error; other lengths outside [max(1, T), max_len] raise
 * DA_DEV_ERR_LEN_RANGE as in decode_attn_run (out 0, lse -inf). Always two kernels (the split
 * kernel with every segment's partial kept, then the combine, which writes out and lse); the
 * workspace is decode_attn_run's (da_workspace_size). With T > 1 the causal bound of query t
 * counts this shard's rows only (row lens[b] - T + t of this cache is the query's own), which
 * is right for the shard holding the sequence's last rows; the earlier shards of a multi-query
 * step would need no mask, which this entry point does not provide.
 */
int decode_attn_run_lse(const da_desc *desc, const void *q, const void *k_cache,
                        const void *v_cache, const int32_t *lens, int32_t max_len,
                        const float *kv_scales, float *out, float *lse, void *workspace,
                        size_t ws_bytes, void *stream);

/*
 * Log-sum-exp merge of `shards` results over disjoint row sets, e.g. the decode_attn_run_lse
 * outputs of the devices that split a context, gathered on one device (same passage as
 * decode_attn_run_lse): with M = max_p lses[p][r] and w_p = exp(lses[p][r] - M),
 *   out[r] = sum_p w_p * outs[p][r] / sum_p w_p,   lse[r] = M + ln sum_p w_p.
 *   outs [shards, rows, d] fp32 (16-byte aligned), lses [shards, rows] fp32,
 *   out  [rows, d] fp32 (16-byte aligned), lse [rows] fp32 or NULL (not wanted).
 * rows >= 0 (any number of query rows, e.g. batch * h_q), d a positive multiple of 4 up to
 * 4096, 1 <= shards <= 4096. A row that no shard holds (every lse -inf) gets out 0 and
 * lse -inf. One kernel on the stream; out and lse must not overlap the inputs.
 */
int decode_attn_merge_lse(int64_t rows, int32_t d, int32_t shards, const float *outs,
                          const float *lses, float *out, float *lse, void *stream);

/*
 * Measurement helper, not part of the attention path: a plain streaming read of `bytes` bytes
 * at buf (16-byte aligned, bytes a positive multiple of 16) by 512 workgroups, each reading a
 * contiguous chunk with 16-byte non-temporal loads. sink is a device buffer of at least 512
 * floats that receives one data-dependent value per workgroup. Timing it gives the read
 * bandwidth the part sustains for a pure stream, the ceiling against which the split kernel's
 * rate is compared.
 */
int da_stream_read(const void *buf, size_t bytes, float *sink, void *stream);

/* Waits for the stream, then copies the error word into *code (host). For tests and tools. */
int da_read_device_error(const void *workspace, void *stream, int32_t *code);

/* Static text for a DA_* status code. */
const char *da_status_string(int status);

/* Message of the latest failure on the calling thread ("" if none). */
const char *da_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
