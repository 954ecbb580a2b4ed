/*
 * mla.h -- paged Multi-Head Latent Attention (MLA) decode for AMD MI355X (gfx950).
 *
 * What is computed.  For every sequence b, query token i < q_len and head
 * h < num_heads, with L = cache_seqlens[b] and R = q_len * num_heads rows
 * (row r = i * num_heads + h):
 *
 *     k_t      = row(kv_cache[block_table[b][t / page_size]][t % page_size])[0:576]
 *     v_t      = k_t[0:512]
 *     s_t      = softmax_scale * sum_d q[b][i][h][d] * k_t[d]        (d < 576)
 *     lse      = log sum_{t<E} exp(s_t)                               (natural log)
 *     out[:]   = sum_{t<E} exp(s_t - lse) * v_t
 *
 * where row() widens a stored cache row (see mla_kv_dtype_t) and E = L, or, for a causal problem, E = max(0, L - (q_len - 1 - i)): query
 * token i then sits at position L - q_len + i of a context whose last q_len
 * rows are the query tokens' own (multi-token / speculative decode), and sees
 * only the tokens up to and including itself.  A row with E = 0 gets out = 0
 * and lse = -inf.
 *
 * This is standard attention S = Q K^T, P = softmax(S), O = P V ("Core
 * mechanism", FlashMLA-ETAP summary on gist.science), in the absorbed MLA form
 * where every head reads the same 576-wide cached row: 512 latent columns that
 * double as V plus 64 rope columns (16 heads and 576-dim heads as in that
 * page's "Limitations noted by the authors"; low-rank joint compression of the
 * KV cache as in its "Implementation details").  Queries are 1-2 tokens over a
 * context of up to 64K tokens ("Problem statement" on the same page).  The
 * kernels evaluate it in the transposed order the page describes,
 * S^T = K Q^T, P^T = softmax(S^T), O^T = V^T P^T, so the context length is the
 * large matrix dimension and the R query rows the small one.
 *
 * The context of each sequence is split across compute units by a host-side
 * planner (mla_plan); per-split partial results (out normalised over the
 * split, and its lse) are merged by the log-sum-exp rule in a second kernel.
 * Rows t >= L are never used, even if they hold NaN; block_table entries past
 * ceil(L / page_size) are never read.
 *
 * Conventions for every function:
 *   - extern "C", never throws, returns mla_status_t (except the few getters
 *     documented otherwise);
 *   - on any error nothing is launched and no output or workspace byte is
 *     written; mla_last_error() then returns a message for this thread;
 *   - device pointers are plain HIP device addresses; "stream" is a
 *     hipStream_t passed as void* (NULL = the default stream); launches are
 *     asynchronous on that stream;
 *   - the library allocates no device memory; the caller owns every device
 *     buffer (q, kv_cache, block_table, cache_seqlens, out, lse, workspace).
 *
 * bf16 values are IEEE-754 binary32 truncated to the upper 16 bits (bfloat16).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 7

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad shape, negative length, ... */
  MLA_ERR_UNSUPPORTED = 2,        /* valid but not implemented (head dims, R, page size) */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4,                /* a HIP runtime call failed; see mla_last_error() */
  MLA_ERR_PLAN_MISMATCH = 5       /* mla_decode with a workspace that last received another plan's
                                     schedule (or none) through mla_plan_upload */
} mla_status_t;

typedef enum { MLA_DTYPE_BF16 = 0, MLA_DTYPE_FP32 = 1 } mla_dtype_t;

/* Storage of one cached token row.
 *   MLA_KV_BF16      576 bf16 values (1,152 bytes): 512 latent columns, then 64 rope columns.
 *   MLA_KV_FP8_E4M3  656 bytes: bytes [0, 512) the latent columns as OCP FP8 E4M3 codes
 *                    (bias 7, no infinities, S.1111.111 = NaN); bytes [512, 640) the rope
 *                    columns as bf16; bytes [640, 656) four float32 group scales.  Latent
 *                    column c widens to e4m3(code) * 2^(E - 127), E the biased exponent of
 *                    scale c / 128: only the exponent of a scale is used, so power-of-two
 *                    scales are the natural choice (every widened value is then exact in
 *                    bf16); scales must be normal, finite numbers.  An FP8 cache is an
 *                    FP8 latent cache in the sense of the FlashMLA pages; this layout is
 *                    this library's.  */
typedef enum { MLA_KV_BF16 = 0, MLA_KV_FP8_E4M3 = 1 } mla_kv_dtype_t;

/* Shapes of one decode call. */
typedef struct {
  int32_t batch;              /* B >= 1 */
  int32_t q_len;              /* S_q >= 1 query tokens per sequence */
  int32_t num_heads;          /* H >= 1; R = q_len * num_heads must be a multiple of 16, <= 256 */
  int32_t head_dim_qk;        /* must be 576 (512 latent + 64 rope) */
  int32_t head_dim_v;         /* must be 512 */
  int32_t page_size;          /* P: tokens per cache page, a positive multiple of 16 */
  int32_t num_pages;          /* physical pages in kv_cache (dimension 0) */
  int32_t max_pages_per_seq;  /* row stride of block_table, in int32 entries */
  mla_dtype_t out_dtype;      /* dtype of `out`: BF16 (round to nearest even) or FP32 */
  int32_t causal;             /* 0: every query token sees all L tokens; 1: token i sees the
                                 first L - (q_len - 1 - i) (see the definition above) */
  mla_kv_dtype_t kv_dtype;    /* storage of the cache rows (MLA_KV_BF16 or MLA_KV_FP8_E4M3) */
} mla_problem_t;

/* Planner options.  Zero-initialise for defaults. */
typedef struct {
  int32_t num_cus;            /* compute units to plan for; 0 = ask the current HIP device */
  int32_t force_splits;       /* 0 = cost model; k > 0 = cut every sequence into min(k, blocks)
                                 near-equal parts, one work-group each (testing the merge) */
  int32_t rows_per_group;     /* 0 = automatic (128 when R is a multiple of 128, else 64 when R is
                                 a multiple of 64, else with a bf16 cache 32 when R is a multiple
                                 of 32; else 16);
                                 16, 32, 64 or 128 = query rows per work-group (16: the 16-row
                                 kernel in R/16 row groups; 32: the 32-row kernel, bf16 cache
                                 only; 64 and 128: the wide kernel, 32 rows per wave on 32x32 MFMA
                                 tiles, bf16 or FP8 rows; R must be a multiple)
                                 -- a tuning and testing knob; MLA_ERR_UNSUPPORTED for 32 with an
                                 FP8 cache or R not a multiple */
  int32_t reserved[5];        /* must be zero */
} mla_plan_options_t;

/* Read-only summary of a plan (for tests and diagnostics). */
typedef struct {
  int32_t num_workers;        /* work-groups in the split-decode launch that have work */
  int32_t grid_size;          /* work-groups launched (num_workers padded, times row groups) */
  int32_t num_segments;       /* (sequence, token range) pieces over all workers */
  int32_t num_partials;       /* partial-result slots (pieces of split sequences) */
  int32_t num_combine;        /* sequences that need the merge kernel */
  int32_t rows_per_group;     /* query rows one work-group handles (16, 32, 64 or 128) */
  int32_t row_groups;         /* R / rows_per_group */
  int32_t granule;            /* token granularity of split boundaries */
  int64_t max_worker_cost;    /* planner cost units (16-token blocks + per-piece overhead) */
  int64_t min_worker_cost;
  int64_t metadata_bytes;     /* bytes uploaded by mla_plan_upload */
  int64_t workspace_bytes;    /* == mla_plan_workspace_bytes() */
} mla_plan_info_t;

typedef struct mla_plan_s* mla_plan_t;   /* opaque, host memory only */

/* ---- Split-KV schedule.  The pages do not describe one: splitting each sequence's context
 * over the compute units is this library's answer to the long-context bandwidth pressure of
 * decode with a short query ("Problem statement", FlashMLA-ETAP summary), where one sequence
 * alone must keep every compute unit streaming.  The schedule, its workspace and the merge of
 * split results are this library's; the merge follows from the online-softmax identity
 * (section 三 of the juejin.cn FlashMLA explainer).
 *
 * mla_plan: build a schedule for `problem` and the given context lengths.
 * Host only; launches nothing.  cache_seqlens_host: B int32 values, each in
 * [0, max_pages_per_seq * page_size].  The plan copies everything it needs and gets an id
 * of its own.  A plan is valid for the same problem and the same cache_seqlens values. */
mla_status_t mla_plan(const mla_problem_t* problem, const int32_t* cache_seqlens_host,
                      const mla_plan_options_t* options /* may be NULL */, mla_plan_t* plan_out);

mla_status_t mla_plan_get_info(mla_plan_t plan, mla_plan_info_t* info);

/* Copy the plan's pieces as int32 quadruples (seq, tok_begin, tok_end, slot; slot -1 =
 * written straight to out/lse) in work-group order, followed by nothing else.
 * `worker_offsets` (num_workers + 1 entries, may be NULL) receives each
 * work-group's first piece index.  Capacities are in int32 elements. */
mla_status_t mla_plan_get_segments(mla_plan_t plan, int32_t* segments, int64_t segments_capacity,
                                   int32_t* worker_offsets, int64_t offsets_capacity);

/* Device workspace the caller must provide to mla_plan_upload / mla_decode
 * (schedule + fp32 partial results + a status word).  Returns 0 for a NULL plan. */
size_t mla_plan_workspace_bytes(mla_plan_t plan);

/* Copy the schedule and the plan's id into `workspace` (device, >= mla_plan_workspace_bytes
 * bytes, 256-B aligned) and clear its status word, asynchronously on `stream`.  Must run
 * once before the first mla_decode with this plan and workspace; the plan must stay alive
 * until the copy has completed on the stream.  The library records (host side) which plan
 * each workspace address last received. */
mla_status_t mla_plan_upload(mla_plan_t plan, void* workspace, size_t workspace_bytes, void* stream);

/* Paged MLA decode (two launches on `stream`: split decode, then the merge of
 * split sequences): the computation defined at the top of this file.
 *   q             [B, q_len, H, 576] bf16, contiguous, 16-B aligned
 *   kv_cache      [num_pages, page_size, row] rows of problem->kv_dtype (1,152 or 656 bytes),
 *                 contiguous, 16-B aligned
 *   block_table   [B, max_pages_per_seq] int32; entries < ceil(L_b/page_size) must lie in
 *                 [0, num_pages).  An entry outside that range is not dereferenced: its
 *                 tokens are dropped and the workspace status word gets bit 0 set.
 *   cache_seqlens [B] int32 on the device, the values the plan was made with (a smaller
 *                 device value shortens the context; a larger one is clipped to the plan's
 *                 and sets bit 2 of the workspace status word)
 *   softmax_scale multiplies q . k before the softmax
 *   out           [B, q_len, H, 512] of problem->out_dtype, 16-B aligned
 *   lse           [B, q_len, H] fp32 natural-log LSE, or NULL
 *   workspace     as uploaded by mla_plan_upload for this plan: MLA_ERR_PLAN_MISMATCH (and no
 *                 launch) when the host record says the address last received another plan,
 *                 or none.  The kernels also compare the id stored in the workspace with the
 *                 plan's (which covers a captured graph replayed after another upload): on a
 *                 mismatch nothing is read from the schedule, out and lse are left untouched
 *                 and bit 3 of the status word is set.
 * Sequences with L = 0 get out = 0 and lse = -inf.
 * Calls that share a workspace must not overlap in time. */
mla_status_t mla_decode(mla_plan_t plan, const void* q, const void* kv_cache,
                        const int32_t* block_table, const int32_t* cache_seqlens,
                        float softmax_scale, void* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Launch only some of mla_decode's kernels (profiling aid): stages is a bit mask,
 * MLA_STAGE_SPLIT runs the split-decode kernel, MLA_STAGE_MERGE the merge of split
 * sequences (which reads the partials the last split stage wrote).
 * mla_decode == mla_decode_stages(..., MLA_STAGE_ALL).  Same arguments and errors
 * as mla_decode; stages outside MLA_STAGE_ALL is MLA_ERR_INVALID_ARGUMENT.
 *
 * MLA_STAGE_COMBINED (alone): one launch instead of two -- the split-decode kernel combines
 * split sequences itself, the way the pages' single-work-group pipeline (FlashMLA-ETAP
 * summary, "Implementation details") finishes a head group within one kernel.  Each piece's
 * partial result is stored with device-scope (write-through) stores;
 * the work-group that completes a (sequence, row group) last, elected by a device-scope
 * counter in the workspace, reads the partials back with device-scope loads and writes out
 * and lse; the counter is back at zero when the launch ends (mla_plan_upload writes zeros).
 * Plans with 16 rows per group only (else MLA_ERR_UNSUPPORTED).  Results equal
 * MLA_STAGE_ALL's up to the order of the combine's additions. */
#define MLA_STAGE_SPLIT 1u
#define MLA_STAGE_MERGE 2u
#define MLA_STAGE_ALL 3u
#define MLA_STAGE_COMBINED 4u
mla_status_t mla_decode_stages(mla_plan_t plan, const void* q, const void* kv_cache,
                               const int32_t* block_table, const int32_t* cache_seqlens,
                               float softmax_scale, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream,
                               uint32_t stages);

/* Test aid: write every sequence's logical rows, in token order, to rows_out
 * [sum_b L_b, row bytes] (sequence b starts at row sum_{b'<b} L_b'), using the
 * same page walk as mla_decode (the block table of PagedAttention, listed under "Builds on"
 * on the mlsanity.com page of the FlashMLA-ETAP paper: token t of sequence b is row
 * t % page_size of page block_table[b][t / page_size]).  Bit-exact copy of the stored rows;
 * async on `stream`.  Entries outside [0, num_pages) are skipped (their rows are not written). */
mla_status_t mla_debug_gather(mla_plan_t plan, const void* kv_cache, const int32_t* block_table,
                              void* rows_out, void* stream);

/* ---- Device-scheduled decode (no host plan; graph-capturable with changing lengths).
 * Not on the pages: the split-KV schedule above, computed by the kernels themselves, for
 * callers that capture the decode in a graph while the lengths change.
 *
 * The work-groups cut the batch's 16-token blocks among themselves at run time from the
 * device cache_seqlens (with W = min(num_workers, T / 4), at least 1, work-group w < W takes
 * blocks [floor(wT/W), floor((w+1)T/W)) of the batch's T blocks, in sequence order); each
 * sequence's first piece records how the sequence was cut, and a second launch combines
 * the pieces of split sequences by log-sum-exp.  The lengths may change between calls
 * (and between replays of a captured graph) up to max_pages_per_seq * page_size (larger
 * device values are clipped to it).  Problems run as 16-row groups.
 *
 * num_workers: work-groups per row group; 0 = the current device's compute units divided
 * by the number of row groups (R / 16), at least 1.
 *
 * Workspace: mla_devplan_workspace_bytes bytes, 256-B aligned; mla_devplan_prepare clears
 * its status word (and need only be called once).  Calls that share a workspace must not
 * overlap in time. */
size_t mla_devplan_workspace_bytes(const mla_problem_t* problem, int32_t num_workers);   /* 0 on error */
mla_status_t mla_devplan_prepare(const mla_problem_t* problem, int32_t num_workers, void* workspace,
                                 size_t workspace_bytes, void* stream);
mla_status_t mla_decode_devplan(const mla_problem_t* problem, int32_t num_workers, const void* q,
                                const void* kv_cache, const int32_t* block_table, const int32_t* cache_seqlens,
                                float softmax_scale, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);

/* mla_decode_devplan in one launch: the split-decode work-groups combine split sequences
 * themselves, as MLA_STAGE_COMBINED does for a host plan (device-scope partial stores and
 * loads, one device-scope counter per (sequence, row group) in the workspace, which
 * mla_devplan_prepare clears and every launch leaves at zero).  Same arguments, workspace
 * and errors as mla_decode_devplan; graph-capturable in the same way. */
mla_status_t mla_decode_devplan_combined(const mla_problem_t* problem, int32_t num_workers, const void* q,
                                         const void* kv_cache, const int32_t* block_table,
                                         const int32_t* cache_seqlens, float softmax_scale, void* out, float* lse,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* The device-scheduled decode for callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid allocation): the same computation and
 * kernels as mla_decode_devplan, with its workspace taken from a scratch array the library
 * holds in device memory, MLA_NOALLOC_SCRATCH_BYTES per GPU, from the first call on that GPU
 * until the process ends.  Nothing is allocated (no hipMalloc, no hipFree); the caller passes
 * inputs and outputs only.  A problem whose device schedule needs more scratch than that
 * (mla_devplan_workspace_bytes(problem, num_workers) > MLA_NOALLOC_SCRATCH_BYTES; with
 * num_workers = 0 on a 256-CU MI355X it needs about 16.8 MB plus 16 bytes per sequence) is
 * refused with MLA_ERR_WORKSPACE_TOO_SMALL before any launch.  Every call on a GPU uses that
 * GPU's one array: calls that overlap in time on one GPU (two streams, two threads) race and
 * must not be made.  Its status word is not reported. */
#define MLA_NOALLOC_SCRATCH_BYTES (24u << 20)
mla_status_t mla_decode_devplan_noalloc(const mla_problem_t* problem, int32_t num_workers, const void* q,
                                        const void* kv_cache, const int32_t* block_table,
                                        const int32_t* cache_seqlens, float softmax_scale, void* out, float* lse,
                                        void* stream);

/* ---- The steps on either side of the decode (an absorbed MLA attention layer).
 *
 * Low-rank joint KV compression (FlashMLA-on-Ascend post, the compression principle and its
 * computation flow): with the shared latent rows c_t, head h's keys and values are
 * K_h = c W_UK[h] and V_h = c W_UV[h].  The decode above runs on the absorbed form
 * (FlashMLA-ETAP summary, "Implementation details"): W_UK is folded into the query and W_UV
 * is applied to the decode's 512-wide latent output, which gives the same attention as the
 * decompressed keys and values.  Per head: 128 query columns before absorption, 64 rotary
 * columns, 128 output columns.
 *
 * Rotary embedding (the pages do not spell out its form; this library's reading): the 64
 * rope columns x rotate in consecutive pairs, (x[2i], x[2i+1]) by the angle
 * pos * rope_base^(-2i/64), evaluated in float64 and rounded once to bf16.
 *
 * Token n = b * q_len + s; positions [B, q_len] int32 on the device gives each new token's
 * position in its sequence (for the decode's causal reading, L_b - q_len + s with L_b
 * counting the new tokens).  `problem` is the decode problem these calls surround, checked
 * as mla_plan checks it.  Every pointer is a device address; launches are asynchronous on
 * `stream`; nothing is allocated. */

/* Query preparation: q_out[n][h] = [W_UK[h] q_nope[n][h] (512), rope(q_pe[n][h], positions[n]) (64)].
 *   q_nope [B, q_len, H, 128] bf16, 16-B aligned     q_pe [B, q_len, H, 64] bf16, 4-B aligned
 *   w_uk   [H, 512, 128] bf16 (row e of head h maps the 128 query columns to latent column e)
 *   q_out  [B, q_len, H, 576] bf16, the decode's q; latent columns are fp32 sums rounded to
 *          nearest even. */
mla_status_t mla_q_absorb(const mla_problem_t* problem, const void* q_nope, const void* q_pe, const void* w_uk,
                          const int32_t* positions, float rope_base, void* q_out, void* stream);

/* Cache append: writes new token n's row at row positions[n] % page_size of page
 * block_table[b][positions[n] / page_size], in problem->kv_dtype's layout:
 *   bf16: [c_kv[n] (512, copied bit for bit), rope(k_pe[n], positions[n]) (64)];
 *   fp8:  latent group g (columns 128g .. 128g+127) as E4M3 codes (nearest, ties to even) of
 *         x / 2^e_g, e_g the smallest integer >= -126 with max|x| <= 448 * 2^e_g (0 for an
 *         all-zero group), scale 2^e_g stored as float32; rope columns as for bf16.
 *   c_kv [B, q_len, 512] bf16, 16-B aligned        k_pe [B, q_len, 64] bf16, 4-B aligned
 *   block_table [B, max_pages_per_seq] int32; kv_cache as for mla_decode.
 * A token whose position is outside [0, max_pages_per_seq * page_size) or whose page entry is
 * outside [0, num_pages) is not written, and bit 1 of *status is set (status: a device int32,
 * or NULL).  Two tokens with the same row race. */
mla_status_t mla_kv_append(const mla_problem_t* problem, const void* c_kv, const void* k_pe,
                           const int32_t* positions, const int32_t* block_table, float rope_base, void* kv_cache,
                           int32_t* status, void* stream);

/* Output projection: o[n][h] = W_UV[h] out_latent[n][h].
 *   out_latent [B, q_len, H, 512] of problem->out_dtype (mla_decode's out), 16-B aligned
 *   w_uv       [H, 128, 512] bf16 (row v of head h maps the latent columns to output column v)
 *   o          [B, q_len, H, 128] of problem->out_dtype, 16-B aligned
 * Products are summed in float32 on bf16 matrix cores; a float32 out_latent enters as
 * bf16(x) + bf16(x - bf16(x)), about 16 significant bits. */
mla_status_t mla_out_absorb(const mla_problem_t* problem, const void* out_latent, const void* w_uv, void* o,
                            void* stream);

/* Read the workspace status word (synchronises `stream`); this library's own diagnostic.
 * Bits, each sticky since the last mla_plan_upload (or mla_devplan_prepare):
 *   bit 0 (1): a used block_table entry was outside [0, num_pages); its tokens were dropped;
 *   bit 2 (4): a device cache_seqlens value exceeded the plan's (host schedule only); the
 *              tokens past the plan's length were not attended;
 *   bit 3 (8): the workspace held another plan's schedule (host schedule only); that launch
 *              computed nothing.
 * Bit 1 is not used here (mla_kv_append's own status word uses it). */
mla_status_t mla_read_status(const void* workspace, void* stream, int32_t* status_out);

/* Measurement aid (this library's): read the first num_workgroups * floor(bytes / num_workgroups
 * / 73,728) * 73,728 bytes of `buffer` (device, 1 KiB aligned) into LDS with the decode's own
 * non-temporal 16-byte global->LDS loads, each work-group its contiguous share, computing nothing:
 * the read ceiling the decode's KV stream is compared with.  Async on `stream`. */
mla_status_t mla_stream_probe(const void* buffer, size_t bytes, int32_t num_workgroups, void* stream);

void mla_plan_destroy(mla_plan_t plan);            /* NULL is a no-op */
const char* mla_status_string(mla_status_t status); /* static string */
const char* mla_last_error(void);                  /* thread-local detail of the last failure */
int32_t mla_abi_version(void);                     /* MLA_ABI_VERSION */

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
