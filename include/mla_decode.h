/*
 * libmla_decode -- paged multi-head latent attention (MLA) decode for MI355X (gfx950).
 *
 * What one call computes (kernelindex amd-mixed-mla submission 689529, module
 * constants block and custom_kernel; submission 690201, the stage-1 and
 * reduce calls):
 *
 *   for every sequence b, its query tokens t = qo_indptr[b] + tau and its
 *   rows  j_0, j_1, ...  (page kv_indices[i], i in [kv_indptr[b], kv_indptr[b+1]),
 *                         slot 0 .. page_size-1 of it; the last page holds
 *                         kv_last_page_len[b] rows):
 *     s_i   = sm_scale * q_scale * kv_scale * sum_{d<576} q[t,h,d] * kv[j_i,d]
 *             (then cap * tanh(s_i / cap) when params.logit_cap = cap > 0)
 *     out[t,h,e] = kv_scale * sum_i softmax(s)_i * kv[j_i,e]     (e < 512)
 *
 * for all 16 heads h, the softmax over the rows token tau sees: all of them,
 * or with MLA_FLAG_CAUSAL the first n - q_len + 1 + tau of the sequence's n
 * rows when it has q_len tokens.  The single latent KV head is 576 wide (512
 * latent + 64 rope); V is the first 512 dims of the same row.  The pages' own
 * calls use page size 1 and one token per sequence; pages of 2 and 8 rows,
 * last-page lengths, q_seq_len, is_causal and logit_cap are the further
 * arguments they pass (submissions 598454, 641982 and 689529).
 *
 * Layouts (all row-major, contiguous, device memory unless stated):
 *   q          [total_q, 16, 576]   bf16 or fp8 e4m3fn (bf16 also with fp8 q_dtype
 *                                   when MLA_FLAG_FUSED_Q_CAST is set)
 *   kv         [pool_pages * page_size, 576]
 *                                   bf16 or fp8 e4m3fn (one KV head); page p is
 *                                   rows p*page_size .. p*page_size+page_size-1
 *   qo_indptr  [batch + 1]          int32, query rows of sequence b
 *   kv_indptr  [batch + 1]          int32, index positions (pages) of sequence b
 *   kv_indices [kv_indptr[batch]]   int32, pool page of each index position
 *   kv_last_page_len [batch]        int32, rows in each sequence's last page
 *                                   (mla_decode_run_paged only; values are
 *                                   clamped into [1, page_size])
 *   out        [total_q, 16, 512]   bf16
 *   lse_out    [total_q, 16]        float32, optional (NULL: not written):
 *                                   the natural-log sum-exp of each token's
 *                                   scores, log sum_i exp(s_i), over the rows
 *                                   it sees; -inf where it sees none
 *   q_scale, kv_scale               one float32 each, in device memory
 *                                   (read only for fp8 operands; may be NULL
 *                                   for bf16 operands)
 *
 * Alignment: q, kv and out must be 16-byte aligned (the kernels move them in
 * 16-byte pieces; every row is a multiple of 16 bytes), the index arrays,
 * scales and lse_out 4-byte aligned.  A misaligned pointer is
 * MLA_ERR_INVALID_ARG.
 *
 * Supported dtype pairs (q, kv): (bf16, bf16), (bf16, fp8), (fp8, fp8).
 * fp8 is the OCP e4m3fn format (max 448, no infinities).
 *
 * Ownership and threading: the caller owns every buffer, the workspace
 * included.  The library never allocates device memory and never
 * synchronises a stream; all work is enqueued on the stream passed in.
 * One workspace must not be used by two calls that may overlap in time
 * (e.g. on two streams): the calls share its partial buffers and counters.
 * A run (mla_decode_run, mla_decode_run_paged, or the attend / merge pair)
 * may be captured into a HIP graph: it enqueues kernels only (no memset, no
 * allocation, no host synchronisation), and the replayed kernels read the
 * index arrays at replay time, so sequence lengths may change in place
 * between replays.
 *
 * Errors: every entry point returns mla_status.  Arguments are validated on
 * the host before any HIP call; a rejected call enqueues nothing.  A HIP
 * launch failure is reported as MLA_ERR_HIP.  Index values (kv_indices,
 * qo_indptr, kv_last_page_len) are not checked on the device: out-of-range
 * values are a caller error and lead to undefined results.  Pool rows
 * (page * page_size + slot) must fit in int32.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_DECODE_ABI_VERSION 4

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent params */
  MLA_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels implement */
  MLA_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned */
  MLA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} mla_status;

typedef enum { MLA_DTYPE_BF16 = 0, MLA_DTYPE_FP8_E4M3FN = 1 } mla_dtype;

/* Flags for mla_decode_params.flags. */
#define MLA_FLAG_FUSED_MERGE 1u /* merge split partials in the last arriving
                                   workgroup of each split sequence instead of
                                   a second launch.  Correct on any device, but
                                   slower on MI355X: the device-scope release /
                                   acquire it needs writes back and invalidates
                                   the per-XCD L2 in every split workgroup. */
#define MLA_FLAG_FUSED_Q_CAST 2u /* with q_dtype = fp8: `q` holds bf16 values and
                                    the attention kernel casts them to fp8
                                    e4m3fn itself, bit-identically to
                                    mla_decode_quantize_q (saves its launch) */
#define MLA_FLAG_CAUSAL 4u /* several query tokens per sequence: token tau of q_len
                              sees the sequence's first n - q_len + 1 + tau rows
                              (submission 689529 builds its metadata with
                              is_causal set) */

/*
 * Problem description.  The fixed fields restate the model constants of
 * submission 689529 (16 heads, 1 KV head, 576 / 512 dims); anything else is
 * MLA_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t batch;        /* sequences, >= 1 */
  int32_t total_q;      /* query rows, in [batch, batch * max_q_len] */
  int32_t num_heads;    /* 16 */
  int32_t num_kv_heads; /* 1 */
  int32_t qk_dim;       /* 576 */
  int32_t v_dim;        /* 512 */
  int32_t page_size;    /* rows per page: a power of two, 1 .. 1024 */
  int32_t q_dtype;      /* mla_dtype */
  int32_t kv_dtype;     /* mla_dtype */
  int32_t num_units;    /* 0 = the device's compute-unit count.  Upper bound on the
                           workgroups that split the KV rows; each one owns a
                           contiguous share of all sequences' rows. */
  int32_t min_chunk;    /* 0 = default (64).  Smallest share of KV rows per workgroup;
                           must be a multiple of 32 when set. */
  uint32_t flags;       /* MLA_FLAG_* */
  int32_t max_q_len;    /* 0 = 1.  Most query tokens of one sequence (qo_indptr[b+1] -
                           qo_indptr[b]), at most 16.  Tokens past it are not
                           computed.  With more than one, each KV tile the
                           kernel reads serves two tokens at once. */
  float logit_cap;      /* 0 = off; > 0: scores pass through cap * tanh(s / cap) */
} mla_decode_params;

/*
 * A plan: validated parameters plus the workspace carve-up.  Plain data; it
 * may be copied.  It stays valid as long as its workspace is alive.  It does
 * not depend on the contents of kv_indptr: the split of KV rows over
 * workgroups is recomputed on the device by every mla_decode_run from the
 * kv_indptr passed to it, so sequence lengths may change between calls.
 */
typedef struct {
  mla_decode_params params; /* with num_units / min_chunk resolved */
  void* workspace;
  size_t workspace_bytes;
  int32_t device;
  int32_t reserved;
  uint64_t off_counters; /* int32 [batch]: arrivals per split sequence (fused merge), left at 0 after each
                            run; then 8 int32: the split of the last attention launch, for the merge */
  uint64_t off_part_o;   /* float32 [(2 * num_units + batch * S) * max_q_len, 16, 512]: normalised split
                            partials; S = min(16, num_units / batch) if num_units >= 2 * batch,
                            else 0: slots per sequence that the merge loads before it reads the
                            split */
  uint64_t off_part_lse; /* float32 [(2 * num_units + batch * S) * max_q_len, 16]: log2-sum-exp of each */
} mla_decode_plan_t;

/*
 * Bytes of device workspace mla_decode_plan needs for these params; 0 if the
 * params are invalid or the device cannot be queried.  This is the sizing
 * half of the pages' per-shape cache (kernelindex amd-mixed-mla submission
 * 689529, cache builder: get_mla_metadata_info_v1 returns the sizes of the
 * metadata and work buffers, which are allocated once per shape; submission
 * 690201 adds the stage-1 intermediates `logits` and `attn_lse` to that
 * cache).  Here the workspace holds the split partials (float32 O and
 * log-sum-exp, the counterparts of logits / attn_lse) and a few counters; no
 * metadata buffer is needed because the split is computed in every launch.
 */
size_t mla_decode_workspace_size(const mla_decode_params* params);

/*
 * Validate params, resolve defaults against the current HIP device, carve
 * the workspace and zero its counters (one small kernel on `stream`).
 * workspace: device memory of at least mla_decode_workspace_size(params)
 * bytes, 256-byte aligned, owned by the caller.  On success *plan is filled.
 *
 * This replaces the pages' metadata call (kernelindex amd-mixed-mla
 * submission 689529, cache builder: get_mla_metadata_v1 turns qo_indptr /
 * kv_indptr / kv_last_page_len into work lists and reduce maps once per
 * shape; submission 598454, metadata builder).  Unlike that call it takes no
 * kv_indptr: the partition of KV rows over workgroups is recomputed on the
 * device from kv_indptr by every attention launch, so the plan stays valid
 * while sequence lengths change.  The plan records the device that was
 * current; later calls with it must run on a stream of that device
 * (MLA_ERR_INVALID_ARG otherwise).
 */
mla_status mla_decode_plan(const mla_decode_params* params, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, mla_decode_plan_t* plan);

/*
 * Enqueue one decode step on `stream` (kernelindex amd-mixed-mla submission
 * 690201: stage-1 split attention then the partial reduce).  The split is
 * chosen on the device from kv_indptr; sequences split over several
 * workgroups are merged by a second launch (or, with MLA_FLAG_FUSED_MERGE, by
 * the last arriving workgroup).  Pointers as in the layout table above;
 * sm_scale is a host float (1/sqrt(576) in the pages).  Every page is full
 * (see mla_decode_run_paged).  Sequences with no KV rows, and causal tokens
 * that see no row, produce zeros.
 */
mla_status mla_decode_run(const mla_decode_plan_t* plan, const void* q, const void* kv,
                          const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                          const float* q_scale, const float* kv_scale, float sm_scale, void* out,
                          hipStream_t stream);

/*
 * The two launches of one decode step, for callers that order or time them
 * separately (the pages call the stage-1 kernel and the reduce directly,
 * submission 690201).  mla_decode_attend enqueues the split attention: it
 * writes the rows of sequences that one workgroup finishes, and the float32
 * partials of split sequences into the workspace (merged in the same launch
 * with MLA_FLAG_FUSED_MERGE).  mla_decode_merge enqueues the merge of those
 * partials into `out` (nothing with MLA_FLAG_FUSED_MERGE); it must follow
 * mla_decode_attend on the same stream with the same plan, qo_indptr,
 * kv_indptr and out, before the workspace is used again: it reads the split
 * that launch chose from the workspace.  Before any mla_decode_attend on a
 * plan's workspace it writes nothing; a sequence that does not fit the split
 * found there (another kv_indptr) is skipped, never read out of bounds.
 * Arguments as for mla_decode_run_paged, which is these two calls in order;
 * both must get the same lse_out (or both NULL): the attention launch writes
 * it for the sequences it finishes, the merge for the split ones.
 */
mla_status mla_decode_attend(const mla_decode_plan_t* plan, const void* q, const void* kv,
                             const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                             const int32_t* kv_last_page_len, const float* q_scale, const float* kv_scale,
                             float sm_scale, void* out, float* lse_out, hipStream_t stream);
mla_status mla_decode_merge(const mla_decode_plan_t* plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
                            void* out, float* lse_out, hipStream_t stream);

/*
 * mla_decode_run with the rows of each sequence's last page given by
 * kv_last_page_len[b] (device int32 [batch], clamped into [1, page_size];
 * NULL: every page full), as the pages pass kv_last_page_lens next to
 * kv_indptr in pages (submissions 598454 and 641982, pages of 2 and 8 rows),
 * and optionally the final log-sum-exp of every token and head in lse_out
 * (float32 [total_q, 16], natural log; NULL: not written).  That is the
 * output the pages' reduce call leaves unused (submission 690201,
 * custom_kernel: the last argument of mla_reduce_v1 is None).
 */
mla_status mla_decode_run_paged(const mla_decode_plan_t* plan, const void* q, const void* kv,
                                const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                                const int32_t* kv_last_page_len, const float* q_scale, const float* kv_scale,
                                float sm_scale, void* out, float* lse_out, hipStream_t stream);

/*
 * mla_decode_run_paged for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no plan and no caller workspace.  The split partials and
 * counters live in a library-owned array of MLA_NOALLOC_SCRATCH_BYTES in
 * device memory, one per device, which that device holds until the process
 * ends.  params are validated and resolved as mla_decode_plan does (against
 * the current device; `stream` must belong to it); a problem whose
 * workspace would exceed the array (mla_decode_workspace_size(params) >
 * MLA_NOALLOC_SCRATCH_BYTES; the array holds the partials of 256 workgroup
 * shares with one query token, or 128 with two, at any batch) is
 * MLA_ERR_WORKSPACE, before any launch.  The first call on a device looks up the array's device address
 * (no allocation).  Every call on one device shares the array, so calls
 * that may overlap in time on one device (two streams, two threads) race
 * and must not be issued; calls in one stream are ordered.  With
 * MLA_FLAG_FUSED_MERGE each call first clears the arrival counters with a
 * small fill kernel.  Other arguments, layouts and errors as for
 * mla_decode_run_paged.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (26u << 20)
mla_status mla_decode_run_noalloc(const mla_decode_params* params, const void* q, const void* kv,
                                  const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                                  const int32_t* kv_last_page_len, const float* q_scale, const float* kv_scale,
                                  float sm_scale, void* out, float* lse_out, hipStream_t stream);

/*
 * Step a0 for fp8 queries: cast n bf16 values to fp8 e4m3fn with
 * round-to-nearest-even and no saturation (|x| > 464, +-inf and NaN become
 * the NaN code with the input's sign), as the pages cast Q straight to fp8
 * with a unit scale (submission 689529 docstring and custom_kernel).
 * q_bf16 and q_fp8 are device buffers of n elements; they must not overlap.
 */
mla_status mla_decode_quantize_q(const void* q_bf16, void* q_fp8, int64_t n, hipStream_t stream);

/*
 * Step a0 with a per-tensor scale (the amax pass that submission 689529's
 * docstring names as the step it skips):
 *   amax    = max |q| over the finite values of q_bf16,
 *   q_scale = amax / 448 in float32 (1 when amax is 0),
 *   q_fp8   = e4m3fn(q / q_scale), the division in float32 (correctly
 *             rounded), round-to-nearest-even, no saturation; +-inf and
 *             NaN give the NaN code with the input's sign.
 * q_scale (one float32 in device memory) is then the q_scale argument of
 * mla_decode_run.  scratch: device memory of at least
 * MLA_QUANT_DYNAMIC_SCRATCH_BYTES, 4-byte aligned, overwritten.  Two
 * launches on `stream`; n may be 0 (q_scale becomes 1).
 */
#define MLA_QUANT_DYNAMIC_SCRATCH_BYTES 1024
mla_status mla_decode_quantize_q_dynamic(const void* q_bf16, void* q_fp8, float* q_scale, void* scratch,
                                         size_t scratch_bytes, int64_t n, hipStream_t stream);

/*
 * Merge split partials produced elsewhere (e.g. KV shards on other devices):
 * for every sequence b and head h, with p in [part_indptr[b], part_indptr[b+1]),
 *   w_p = exp(lse[p,h] - max_p lse[p,h]),  out[b,h,:] = sum_p w_p o[p,h,:] / sum_p w_p
 * rounded to bf16 (submission 690201: mla_reduce_v1 over logits / attn_lse).
 *   part_o   [n_parts, 16, 512] float32, softmax-normalised over each part
 *   part_lse [n_parts, 16] float32, natural-log sum-exp of each part's scores
 *   out      [batch, 16, 512] bf16
 *   lse_out  [batch, 16] float32 or NULL: log sum_p exp(lse[p,h]), the
 *            natural-log sum-exp over all parts (the reduce's final-LSE
 *            output, which submission 690201 passes as None)
 * Parts with lse = -inf carry no weight and their part_o rows are ignored
 * (they may hold NaN, e.g. 0/0 of an empty shard); a sequence whose parts
 * are all empty (or that has none) gets zeros and lse -inf.  A NaN lse makes
 * that head's output and lse NaN.  part_o and out
 * must be 16-byte aligned, part_lse, part_indptr and lse_out 4-byte aligned.
 */
mla_status mla_decode_reduce(const float* part_o, const float* part_lse, const int32_t* part_indptr,
                             int32_t batch, void* out, float* lse_out, hipStream_t stream);

/*
 * Diagnostic, not part of the decode path: read `bytes` of device memory at
 * `buf` once, in one pass of workgroups of 512 threads that each read their
 * own MLA_READ_PROBE_BYTES_PER_WORD contiguous bytes (four 16-byte
 * non-temporal loads per thread, all in flight together), and store one
 * 32-bit word per workgroup to `sink`: word k is the xor of the 32-bit words
 * in bytes [k * MLA_READ_PROBE_BYTES_PER_WORD, (k + 1) * ...) of `buf`.
 * Timed around its launch, this gives the device's plain streaming read rate
 * for that many bytes, beside which the decode kernels' bandwidth can be set.
 * `buf` must be 16-byte aligned and `bytes` a positive multiple of 16; `sink`
 * must hold at least ceil(bytes / MLA_READ_PROBE_BYTES_PER_WORD) words.
 * Otherwise MLA_ERR_INVALID_ARG, before any launch.
 */
#define MLA_READ_PROBE_BYTES_PER_WORD 32768
mla_status mla_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, hipStream_t stream);

/* Static description of a status code.  Derived: the pages define no error
 * reporting (their calls raise Python exceptions), so no passage backs it. */
const char* mla_status_string(mla_status status);

/* MLA_DECODE_ABI_VERSION of the built library. */
int32_t mla_decode_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
