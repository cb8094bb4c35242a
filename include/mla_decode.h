/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) paged MLA decode library.
 *
 * The operation: multi-head latent attention decode over a paged latent KV
 * cache. Every KV slot holds one latent row of 576 values (512 compressed
 * "nope" dims followed by 64 RoPE dims); all heads attend to the same row and
 * V is its first 512 dims. Pages hold one token each, so a request row names
 * its keys with a flat CSR index list (kv_indptr, kv_indices) -- "one row per
 * request, same index list" ([ROCm][Spec Decode] Add Aiter MLA decode support
 * non-causal draft block, vLLM pull request 53001, Purpose). A request row may
 * carry a block of up to 16 query tokens (qo_indptr): causal for a speculative
 * verify pass, with the mask on global positions (ATOM pull request 2760,
 * Problem), or non-causal for a draft block, the mask being a runtime flag
 * rather than a separate kernel (vLLM pull request 53001, Purpose). Long rows
 * are split across workgroups by a host-built split plan ([DSV4] Tuned ASM
 * FP8 decode with split plans, ATOM pull request 2462, Summary part 1) or one
 * planned per call from the real lengths (same page, Summary part 2), and the
 * split partials are merged by log-sum-exp (same page, Dependencies: split and
 * merge).
 *
 * Semantics, for request row b with L = kv_indptr[b+1] - kv_indptr[b] keys
 * and q_b = qo_indptr[b+1] - qo_indptr[b] query tokens:
 *   k_j   = pool[kv_indices[kv_indptr[b] + j]] * kv_scale,   j in [0, L)
 *   q     = Q[qo_indptr[b] + i, h] * q_scale
 *   token i sits at position L - q_b + i, key j at position j; causal: token i
 *   sees keys j <= L - q_b + i; non-causal: all j < L
 *   s_j   = softmax_scale * (q . k_j)
 *   LSE   = ln sum_visible exp(s_j)        (natural log, fp32)
 *   O     = sum_visible exp(s_j - LSE) * k_j[0:512]   (rounded to bf16)
 *   no visible key: O = 0, LSE = -inf.
 *
 * Conventions for every call:
 *   - All integers are int32 unless noted. Device buffers are contiguous.
 *   - The caller owns every buffer. The library never allocates device
 *     memory, never synchronizes the device and keeps no pointer between
 *     calls. All work is enqueued on the caller's stream.
 *   - Every entry point returns an mla_status. A negative value is an error;
 *     mla_last_error() gives the message (thread-local). Arguments are checked
 *     on the host before anything is launched; an error launches nothing.
 *   - Data that lives on the device (index values, indptr monotonicity,
 *     q_b <= q_len_max) cannot be checked without a synchronization and is a
 *     caller contract: kv_indices values in [0, num_slots), kv_indptr and
 *     qo_indptr non-decreasing, qo_indptr[0] = 0, per-row q_b <= q_len_max, and
 *     kv_indptr[b+1] - kv_indptr[b] equal to the kv_lens the plan was built
 *     from. kv_indptr[0] may be non-zero (an offset list; indices are used as
 *     absolute positions in kv_indices). An index outside [0, num_slots)
 *     gives a wrong result but never a read outside the pool: the decode
 *     reads row num_slots - 1 in its place.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point is exported from libmla_decode.so (built with hidden
 * visibility for everything else). */
#define MLA_API __attribute__((visibility("default")))

#define MLA_ABI_VERSION 1
#define MLA_D_LATENT 576   /* latent row: 512 compressed dims + 64 RoPE dims */
#define MLA_D_V 512        /* V = the first 512 latent dims */
#define MLA_MAX_HEADS 128
#define MLA_MAX_Q_LEN 16
#define MLA_MAX_DCP_WORLD 64

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,   /* null pointer, bad enum, misalignment, bad size */
  MLA_ERR_UNSUPPORTED = -2,   /* a shape or dtype outside the supported range */
  MLA_ERR_WORKSPACE = -3,     /* workspace too small for the plan */
  MLA_ERR_PLAN_MISMATCH = -4, /* plan words do not match this call */
  MLA_ERR_HIP = -5            /* a HIP launch reported an error */
} mla_status;

/* Element formats. fp8 is OCP e4m3fn (max 448, no infinities); a stored value
 * times its per-tensor scale is the real value. */
typedef enum { MLA_BF16 = 0, MLA_FP8_E4M3 = 1 } mla_dtype;

/* UNIFORM gives every row the same split count (a plan that depends only on
 * the row count, the longest row and the config); LENGTH_AWARE plans from
 * the real lengths, as the persistent kernel of ATOM pull request 2462,
 * Summary part 2 does. AUTO builds both and keeps the one whose estimated
 * duration is shorter (keys plus a fixed cost per split: UNIFORM's
 * costliest split or its total over the compute units, LENGTH_AWARE's
 * fullest lane), UNIFORM on a tie. */
typedef enum { MLA_PLAN_AUTO = 0, MLA_PLAN_UNIFORM = 1, MLA_PLAN_LENGTH_AWARE = 2 } mla_plan_mode;

/* OR into the plan mode to have split rows (at most 16 splits) merged inside
 * the decode kernel by the last of their splits to finish each 128-row tile,
 * instead of by a second kernel: one launch instead of two. It costs an L2
 * write-back per work item and an L2 invalidation per merged tile (the L2s
 * of the MI355X's eight XCDs are not coherent with each other), and on the
 * measured workloads it is slower than the second kernel; the plan records
 * the request in its header mode word. */
#define MLA_PLAN_MERGE_IN_KERNEL 0x100

/* OR into the plan mode (fp8 KV only) to run the PV products in fp8: P is
 * rounded to e4m3 after a power-of-two scale per (query row, 32-key tile)
 * that puts the tile's largest weight in (128, 256], and the products
 * (v_mfma_scale_f32_32x32x64_f8f6f4, two tiles per product) take that scale
 * back out exactly, so V is never converted. It halves the matrix-core work
 * of PV against the bf16 PV products; the price is P's 4-bit significand
 * (the measured error stays inside the fp8 tolerance, 4e-2 of max|O|). The
 * plan records the request in its header mode word; mla_decode_plan refuses
 * it (UNSUPPORTED) with bf16 KV or together with MLA_PLAN_MERGE_IN_KERNEL. */
#define MLA_PLAN_FP8_PV 0x200

/* Upper bound on the int32 words mla_decode_plan can write for these sizes,
 * so that a caller can size the host plan buffer once (the plan sits next to
 * the decode CSR on the host: ATOM pull request 2462, Summary part 1).
 * Host only; never fails for rows >= 1, heads in [1,128], q_len_max in [1,16],
 * num_cus >= 1. Errors: INVALID_ARG (null words_out, rows or num_cus < 1),
 * UNSUPPORTED (heads or q_len_max out of range). */
MLA_API int32_t mla_decode_plan_capacity(int32_t rows, int32_t num_cus, int32_t num_heads,
                                 int32_t q_len_max, int64_t* words_out);

/* Build the split plan on the host: per request row a split count and
 * split_indptr, built next to the decode CSR, either uniform (the count
 * depends only on the row count, the longest row and the config, so a graph
 * captured with it replays with changing lengths) or planned per call from
 * the real lengths (ATOM pull request 2462, Summary parts 1 and 2). Pure:
 * the same inputs give the same words. kv_lens: host [rows], each >= 0.
 * num_cus: the device's compute-unit count (256 on MI355X). plan: host buffer
 * of plan_words int32, caller-owned; on success word 19 holds the number of
 * words written.
 *
 * Plan words (spec version 4): a 20-word header [magic 0x4D4C4150, version 4,
 * rows, heads, q_len_max, kv_dtype, num_cus, mode_used, M_UNIT (128), u,
 * N_MAX (256), MIN_SPLIT_KEYS, ITEM_OVERHEAD, OCC, S, W, G, P, 20,
 * total_words], then split_indptr[rows+1], split_row[S], split_begin[S],
 * split_end[S], split_part[S], work_indptr[G+1], item_split[W], item_m[W].
 * S splits, W work items (split, M tile of 128 query rows: row r of a request
 * row's block is token r / heads, head r % heads), G workgroups, P
 * partial-buffer slots. mode_used is UNIFORM or LENGTH_AWARE (AUTO resolved;
 * | MLA_PLAN_MERGE_IN_KERNEL and | MLA_PLAN_FP8_PV when asked). Errors:
 * INVALID_ARG (null, negative length, too few words, unknown dtype or mode,
 * num_cus < 1), UNSUPPORTED (heads, q_len_max or rows out of range, total
 * length above 2^31 - 1, MLA_PLAN_FP8_PV with bf16 KV or with
 * MLA_PLAN_MERGE_IN_KERNEL). */
MLA_API int32_t mla_decode_plan(const int32_t* kv_lens, int32_t rows, int32_t num_heads,
                        int32_t q_len_max, mla_dtype kv_dtype, mla_plan_mode mode,
                        int32_t num_cus, int32_t* plan, int64_t plan_words);

/* Workspace bytes mla_decode_fwd needs for this plan (the per-device
 * workspace that holds split partials until they are merged: ATOM pull
 * request 2462, Summary part 1 and Dependencies): 0 when no row is split,
 * else the partials (bf16 O, fp32 LSE), P * q_len_max * heads * (512 * 2 + 4)
 * bytes, preceded for an MLA_PLAN_MERGE_IN_KERNEL plan by 256 KiB of
 * split-arrival counters. plan: host words from mla_decode_plan. Errors:
 * INVALID_ARG (null), PLAN_MISMATCH (bad magic, version or header). */
MLA_API int32_t mla_decode_workspace_size(const int32_t* plan, int64_t* bytes_out);

/* For an MLA_PLAN_MERGE_IN_KERNEL plan: zero the workspace's counter region
 * (its first 256 KiB). Call once after allocating a workspace (or allocate it
 * zeroed); every completed mla_decode_fwd leaves the region zero again, so
 * one workspace serves any number of later calls and plans. Enqueued on
 * `stream` as a kernel (no memset), so it may also be captured in a graph.
 * Other plans need no initialization (nothing is launched). Errors:
 * INVALID_ARG, PLAN_MISMATCH, WORKSPACE (too small for this plan), HIP. */
MLA_API int32_t mla_decode_workspace_init(const int32_t* plan, void* workspace,
                                          int64_t workspace_bytes, void* stream);

/*
 * Enqueue the decode: one decode kernel over the plan's G workgroups, then,
 * if any row is split, one merge kernel (with an MLA_PLAN_MERGE_IN_KERNEL
 * plan, rows with at most 16 splits are merged inside the decode kernel, the
 * split-and-merge of the persistent kernel of ATOM pull request 2462,
 * Dependencies, and the merge kernel only runs for rows with more). No host
 * synchronization.
 * A UNIFORM plan takes each split's key range from the live lengths
 * (split k of n covers [k L / n, (k + 1) L / n) of L = kv_indptr[b+1] -
 * kv_indptr[b]), so a plan built once stays valid when the lengths change:
 * a call captured in a graph can be replayed after the index lists are
 * updated in place (rows, q_len_max and the plan words fixed).
 *   q          device, [qo_indptr[rows], num_heads, 576] of q_dtype, 16-byte aligned
 *   q_scale    device float scalar, or NULL for 1.0 (fp8 Q needs its scale)
 *   kv_pool    device, [num_slots, 576] of kv_dtype, 16-byte aligned
 *   kv_scale   device float scalar, or NULL for 1.0
 *   qo_indptr  device [rows+1];  kv_indptr device [rows+1];  kv_indices device
 *              (q, kv_indices, o and lse are never NULL; when they have no
 *              entries -- every query block or every row empty -- any valid
 *              device address will do, since nothing there is read or written)
 *   plan_host  host words from mla_decode_plan; plan_dev a device copy of the
 *              same words (the caller uploads it, e.g. from pinned memory)
 *   causal     0 = non-causal, 1 = causal on positions (see top of file)
 *   softmax_scale  finite and > 0
 *   o          device bf16 [qo_indptr[rows], num_heads, 512], 16-byte aligned
 *   lse        device fp32 [qo_indptr[rows], num_heads]
 *   workspace  device, >= mla_decode_workspace_size bytes, 16-byte aligned
 *              (may be NULL when that size is 0), its counter region zero
 *              (mla_decode_workspace_init); the rest is scratch. Calls that
 *              overlap on one workspace race
 *   stream     hipStream_t (NULL = the default stream)
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, PLAN_MISMATCH (plan header
 * differs from rows / num_heads / q_len_max / kv_dtype, or a plan from a
 * different spec version), HIP (launch failure).
 */
MLA_API int32_t mla_decode_fwd(const void* q, mla_dtype q_dtype, const float* q_scale,
                       const void* kv_pool, mla_dtype kv_dtype, const float* kv_scale,
                       int64_t num_slots, const int32_t* qo_indptr, const int32_t* kv_indptr,
                       const int32_t* kv_indices, const int32_t* plan_host,
                       const int32_t* plan_dev, int32_t rows, int32_t num_heads,
                       int32_t q_len_max, int32_t causal, float softmax_scale, void* o,
                       float* lse, void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of the library-owned scratch that mla_decode_fwd_noalloc uses per GPU. */
#define MLA_NOALLOC_SCRATCH_BYTES (64LL << 20)

/*
 * mla_decode_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under graph capture, serving loops that may
 * not call the allocator, harnesses that forbid hipMalloc. The split partials
 * (and an in-kernel-merge plan's split counters) go to a static device array
 * of MLA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library owns; each GPU the
 * library runs on holds its own copy until the process ends. The call never
 * allocates or frees memory. The caller still owns and passes the inputs and
 * outputs; arguments and results are those of mla_decode_fwd (the same
 * kernels run, so the outputs are bit-identical for the same plan).
 * Every call on one GPU shares that GPU's array and the array keeps the last
 * call's contents: calls that overlap on one GPU (two streams, two threads)
 * race and must be ordered by the caller. For an in-kernel-merge plan the
 * call first clears the counters it uses with a fill kernel (no memset), so
 * the call may be captured in a graph.
 * Errors: those of mla_decode_fwd, and WORKSPACE when the plan needs more
 * than MLA_NOALLOC_SCRATCH_BYTES of scratch (mla_decode_workspace_size
 * gives the need; use mla_decode_fwd with a caller workspace then), HIP when
 * the scratch's device address cannot be looked up.
 */
MLA_API int32_t mla_decode_fwd_noalloc(const void* q, mla_dtype q_dtype, const float* q_scale,
                                       const void* kv_pool, mla_dtype kv_dtype,
                                       const float* kv_scale, int64_t num_slots,
                                       const int32_t* qo_indptr, const int32_t* kv_indptr,
                                       const int32_t* kv_indices, const int32_t* plan_host,
                                       const int32_t* plan_dev, int32_t rows, int32_t num_heads,
                                       int32_t q_len_max, int32_t causal, float softmax_scale,
                                       void* o, float* lse, void* stream);

/*
 * Decode of one decode-context-parallel (DCP) shard. With dcp_world ranks the
 * KV of a row is dealt round-robin: rank dcp_rank holds the keys whose global
 * position is dcp_rank, dcp_rank + dcp_world, ..., so its local key j (the
 * j-th entry of its own index list) sits at global position
 * j * dcp_world + dcp_rank. A q_b-token block at the end of a row of
 * P = kv_len_global[b] keys in total has token i at global position
 * P - q_b + i, and the causal mask is taken on global positions (ATOM pull
 * request 2760, Problem): local key j is visible iff
 * j * dcp_world + dcp_rank <= P - q_b + i. Non-causal blocks see every local
 * key. The result is this shard's (O_r, LSE_r) per (token, head); the
 * shards' results combine with mla_merge_shards.
 * Arguments as mla_decode_fwd (the plan is built from the shard's local
 * lengths), plus:
 *   dcp_world      1..64;  dcp_rank  0..dcp_world-1
 *   kv_len_global  device int32 [rows], P per row (caller contract: the
 *                  shard's local length is the number of positions
 *                  p < P with p mod dcp_world == dcp_rank)
 * dcp_world = 1, dcp_rank = 0 and P = the local length is mla_decode_fwd.
 * Errors: those of mla_decode_fwd, and INVALID_ARG for a bad world, rank or
 * a null kv_len_global.
 */
MLA_API int32_t mla_decode_fwd_dcp(const void* q, mla_dtype q_dtype, const float* q_scale,
                                   const void* kv_pool, mla_dtype kv_dtype, const float* kv_scale,
                                   int64_t num_slots, const int32_t* qo_indptr,
                                   const int32_t* kv_indptr, const int32_t* kv_indices,
                                   const int32_t* plan_host, const int32_t* plan_dev, int32_t rows,
                                   int32_t num_heads, int32_t q_len_max, int32_t causal,
                                   float softmax_scale, void* o, float* lse, void* workspace,
                                   int64_t workspace_bytes, int32_t dcp_world, int32_t dcp_rank,
                                   const int32_t* kv_len_global, void* stream);

/*
 * Log-sum-exp merge of `world` shard results (the combine step of DCP; the
 * same merge as that of split-KV partials):
 *   LSE = ln sum_r exp(LSE_r),  O = sum_r exp(LSE_r - LSE) * O_r  (bf16)
 * shards with LSE_r = -inf are skipped; if all are, O = 0 and LSE = -inf.
 *   o_parts    device bf16 [world, tokens, num_heads, 512], 16-byte aligned
 *              (shard r's mla_decode_fwd_dcp output at index r)
 *   lse_parts  device fp32 [world, tokens, num_heads]
 *   o, lse     device bf16 [tokens, num_heads, 512] (16-byte aligned), fp32
 *              [tokens, num_heads]
 * world 1..64. tokens == 0 launches nothing. Errors: INVALID_ARG, HIP.
 */
MLA_API int32_t mla_merge_shards(const void* o_parts, const float* lse_parts, int32_t world,
                                 int32_t tokens, int32_t num_heads, void* o, float* lse,
                                 void* stream);

/*
 * Test hook: run the decode kernel's own index gather and tile loader over
 * every split of the plan and write the rows it staged in LDS, in the form
 * the matrix cores consume (bf16; fp8 slots converted exactly), to
 * dense_out: device bf16 [kv_indptr[rows] - kv_indptr[0], 576], row
 * kv_indptr[b] - kv_indptr[0] + j for key j of row b. Same argument rules and
 * errors as mla_decode_fwd.
 */
MLA_API int32_t mla_debug_gather(const void* kv_pool, mla_dtype kv_dtype, int64_t num_slots,
                         const int32_t* kv_indptr, const int32_t* kv_indices,
                         const int32_t* plan_host, const int32_t* plan_dev, int32_t rows,
                         void* dense_out, void* stream);

/* Source element formats of the cache writer's inputs. */
typedef enum { MLA_SRC_BF16 = 0, MLA_SRC_FP16 = 1, MLA_SRC_FP32 = 2 } mla_src_dtype;

/*
 * Latent cache write (the step that feeds the decode path: the decode's
 * KV-cache write of vLLM pull request 57942, Details). For t in [0, tokens):
 *   pool[slot_mapping[t]][0:512]   = convert(kv_c[t][0:512])
 *   pool[slot_mapping[t]][512:576] = convert(k_pe[t][0:64])
 * Each source is read at its own declared dtype and converted, never
 * reinterpreted: the review thread of that page traces garbage RoPE columns
 * to an fp32 k_pe tensor written as if it were bf16.
 *   bf16 pool: round to nearest even (NaN stays a NaN).
 *   fp8 pool:  v = x / kv_scale in fp32 (one correctly rounded division),
 *              saturated to +-448, rounded to the nearest e4m3fn value with
 *              ties to the even code; NaN -> 0x7F; zeros keep their sign.
 *   kv_c       device, row t at kv_c + t * kv_c_stride elements (stride >= 512)
 *   k_pe       device, row t at k_pe + t * k_pe_stride elements (stride >= 64)
 *   slot_mapping  device int64 [tokens]; a negative slot (a padding token) and
 *              a slot >= num_slots are skipped (nothing is written)
 *   kv_pool    device [num_slots, 576] of kv_dtype
 *   kv_scale   device float scalar (fp8), or NULL for 1.0
 * Tokens with equal slots race (one of them wins). tokens == 0 launches
 * nothing. Errors: INVALID_ARG (null pointer, bad enum, short stride,
 * misaligned source, num_slots < 1), HIP.
 */
MLA_API int32_t mla_cache_write(const void* kv_c, mla_src_dtype kv_c_dtype, int64_t kv_c_stride,
                                const void* k_pe, mla_src_dtype k_pe_dtype, int64_t k_pe_stride,
                                const int64_t* slot_mapping, int32_t tokens, void* kv_pool,
                                mla_dtype kv_dtype, const float* kv_scale, int64_t num_slots,
                                void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
MLA_API const char* mla_last_error(void);

/* MLA_ABI_VERSION of the built library. */
MLA_API int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
