/*
 * streamkl.h - C ABI of libstreamkl: fused attention KL divergence for AMD
 * Instinct MI355X (gfx950).
 *
 * For every batch b, head h and query row i the library computes the KL
 * divergence between two attention distributions over the same keys,
 *
 *   P1 = softmax(scale1 * Q1 K1^T),   P2 = softmax(scale2 * Q2 K2^T),
 *   KL_i = sum_j P1[i,j] * (log P1[i,j] - log P2[i,j]),
 *
 * without ever holding either N_Q x N_K matrix in memory (StreamKL; agidaily.cc
 * StreamKL article, sections "Online formula" and "Forward: single-pass
 * streaming kernel"; StreamKL paper digest, "Abstract").  The forward returns
 * KL and both log-sum-exp vectors; the two backward calls rebuild P1 and P2
 * tile by tile from the saved LSEs (article section "Backward:
 * recompute-based tile-by-tile gradients").
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensors Q1, K1 (head dim d1) and Q2, K2 (head dim d2) are [B, H, N, d]
 *   with arbitrary element strides for the b, h and n axes (skl_shape) and a
 *   contiguous d axis.  [B, H, N, d] and [B, N, H, d] storage both fit.
 * - Element type: bf16 or fp32 (skl_dtype), the same for all four inputs.
 *   Arithmetic is fp32 (bf16 MFMA products accumulate in fp32).
 * - Per-row vectors (kl, lse1, lse2, dkl) are contiguous fp32 [B, H, N_Q].
 *   LSE and KL are in natural-log units (nats).
 * - Causal masking is bottom-right aligned: row i sees keys
 *   j <= i + (N_K - N_Q); causal calls need N_Q <= N_K.
 * - All pointers except skl_shape are DEVICE pointers owned by the caller.
 *   The library never allocates or frees device memory.  Between calls it
 *   keeps only thread-local host state: the last error message
 *   (skl_last_error) and the profiling events of skl_set_kernel_events.
 * - Every call only enqueues work on `stream` and returns; it never
 *   synchronises.  Calls on one stream run in order.
 * - Validation happens on the host before anything is enqueued; on any
 *   error nothing is enqueued and no output is touched.  A launch failure
 *   reported by the HIP runtime returns SKL_ERR_HIP.
 * - Sizes of zero (B, H or N_Q) are valid and enqueue nothing, with one
 *   exception: a backward call with N_Q = 0 < N_K (and B, H > 0) writes zeros
 *   into its key gradients, which have rows although no query sees them (it
 *   needs only their pointers; the other row and query pointers may be NULL).
 *   N_K = 0 with N_Q > 0 is invalid (an empty softmax).
 * - N_Q and N_K must be below 2^30 and B * H at most 2^31 (row indices are
 *   32-bit inside the kernels); larger sizes return SKL_ERR_UNSUPPORTED.
 *   So does a shape whose kernels would need more than (2^32 - 1) / 256
 *   workgroups in one dispatch (one workgroup per 128 queries or keys of a
 *   head, times the split count where there is one).
 * - Backward calls write each gradient with the strides of its input, so
 *   the optimised side's inputs (all four for skl_backward_joint) must map
 *   distinct elements to distinct addresses: a zero stride on an axis of
 *   size > 1 (e.g. one K broadcast over the heads) or overlapping axes
 *   return SKL_ERR_UNSUPPORTED.  The check takes the axes of size > 1 in
 *   order of increasing stride and needs each stride to reach past the span
 *   of the axes inside it (the d axis spans d elements).  The forward reads
 *   its inputs only and accepts such layouts.
 * - Alignment: data pointers 16-byte aligned; b/h/n strides multiples of 8
 *   elements (bf16) or 4 elements (fp32).  Supported head dims: 64 and 128.
 * - Outputs must not alias inputs.
 */
#ifndef STREAMKL_H
#define STREAMKL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum skl_status {
  SKL_OK = 0,
  SKL_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad scale, causal with N_Q > N_K, ... */
  SKL_ERR_UNSUPPORTED = 2,        /* head dim, dtype or alignment outside what the kernels cover */
  SKL_ERR_WORKSPACE_TOO_SMALL = 3,
  SKL_ERR_HIP = 4                 /* the HIP runtime reported an error for a launch */
} skl_status;

typedef enum skl_dtype { SKL_BF16 = 0, SKL_F32 = 1 } skl_dtype;

/*
 * Backward algorithms.
 *  SKL_BWD_SPLIT (default): one kernel owns keys and writes dK, one owns
 *    queries and writes dQ; both recompute the two logit tiles.  No atomics,
 *    bitwise deterministic.  The workspace is optional: when the query tiles
 *    alone cannot fill the device (few heads x queries, many keys -- the
 *    regime of split-K) and the caller passes skl_backward_workspace_size()
 *    bytes, the dQ kernel splits its keys into ranges whose fp32 partials a
 *    reduce kernel sums; otherwise dQ is written directly.
 *  SKL_BWD_FUSED_ATOMIC: one kernel visits each (query tile, key tile) pair
 *    once, keeps dK on chip and adds dQ into an fp32 workspace with atomics
 *    (article section "GPU kernel optimisations", fused backward); needs
 *    skl_backward_workspace_size() bytes; dQ is not bitwise reproducible.
 */
typedef enum skl_bwd_algo { SKL_BWD_SPLIT = 0, SKL_BWD_FUSED_ATOMIC = 1 } skl_bwd_algo;

/* Problem shape and input layout.  Strides are in elements. */
typedef struct skl_shape {
  int64_t B, H, NQ, NK;
  int32_t d1, d2;       /* head dims of (Q1, K1) and of (Q2, K2) */
  int32_t dtype;        /* skl_dtype of Q1, K1, Q2, K2 */
  int32_t reserved;     /* must be 0 */
  int64_t sq1[3];       /* Q1 strides of the (b, h, n) axes */
  int64_t sk1[3];       /* K1 strides */
  int64_t sq2[3];       /* Q2 strides */
  int64_t sk2[3];       /* K2 strides */
} skl_shape;

/*
 * Forward (one pass).  Streams the key tiles of K1 and K2 once per query
 * tile, keeping per-row running maxima m1, m2, sums l1, l2 and
 * acc = sum_j exp(S1[j] - m1) * (S1[j] - S2[j]) with correction-factor
 * rescaling, and writes only
 *   kl[b,h,i]   = acc / l1 + LSE2 - LSE1,
 *   lse1[b,h,i] = log sum_j exp(S1[i,j]),  lse2 likewise,
 * (article sections "Online formula" and "Forward: single-pass streaming
 * kernel").  scale1, scale2 must be finite and > 0.
 */
skl_status skl_forward(const skl_shape* shape,
                       const void* q1, const void* k1, const void* q2, const void* k2,
                       float scale1, float scale2, int causal,
                       float* kl, float* lse1, float* lse2, hipStream_t stream);

/*
 * Split-K forward: the keys are cut into num_splits contiguous ranges (the
 * split length is rounded up to the kernel's key tile) and each range of
 * each query tile runs as its own workgroup, writing partial statistics to
 * `ws`, for shapes whose query tiles alone cannot fill the GPU (article
 * section "GPU kernel optimisations", split-K).  skl_reduce merges them.
 * ws must hold skl_forward_splitk_workspace_size() bytes, 16-byte aligned;
 * its contents are only meaningful to skl_reduce with the same shape and
 * num_splits.  num_splits >= 1.
 */
size_t skl_forward_splitk_workspace_size(const skl_shape* shape, int num_splits);

skl_status skl_forward_splitk(const skl_shape* shape,
                              const void* q1, const void* k1, const void* q2, const void* k2,
                              float scale1, float scale2, int causal, int num_splits,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Merges the partials of skl_forward_splitk into kl, lse1, lse2 (same
 * meaning as skl_forward).  Only B, H and N_Q of `shape` are used.
 */
skl_status skl_reduce(const skl_shape* shape, int num_splits, const void* ws, size_t ws_bytes,
                      float* kl, float* lse1, float* lse2, hipStream_t stream);

/*
 * Allocation-free split-K forward, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Computes what skl_forward_splitk followed by skl_reduce
 * computes (outputs kl, lse1, lse2 as skl_forward), with the split partials in
 * a static device array of skl_noalloc_scratch_bytes() bytes (32 MiB) that the
 * library holds on each GPU it runs on until the process ends, instead of a
 * caller workspace.  Allocates nothing.  A shape whose partials
 * (20 * B * H * N_Q * num_splits bytes) exceed the array returns
 * SKL_ERR_UNSUPPORTED before anything is enqueued; other errors as
 * skl_forward_splitk and skl_reduce.  Every call on one GPU uses that GPU's
 * array: calls that overlap on one GPU (several streams or host threads)
 * race, and the caller must serialise them.
 */
size_t skl_noalloc_scratch_bytes(void);
skl_status skl_forward_splitk_noalloc(const skl_shape* shape,
                                      const void* q1, const void* k1, const void* q2, const void* k2,
                                      float scale1, float scale2, int causal, int num_splits,
                                      float* kl, float* lse1, float* lse2, hipStream_t stream);

/*
 * Workspace bytes a backward call with algorithm `algo` uses, with
 * d = d2 (teacher == 0) or d1 (teacher != 0):
 *  SKL_BWD_FUSED_ATOMIC: the fp32 dQ accumulator, 4 * B * H * N_Q * d
 *    (required);
 *  SKL_BWD_SPLIT: 0 when B * H * ceil(N_Q / 128) query tiles fill the
 *    current device (two per compute unit), else S * 4 * B * H * N_Q * d for
 *    the S key ranges of the dQ kernel (S <= 64, each range >= 512 keys);
 *    optional, see skl_bwd_algo.  The value depends on the current device's
 *    compute-unit count.
 */
size_t skl_backward_workspace_size(const skl_shape* shape, int teacher, int algo);

/*
 * Backward, "optimise P2" (the student, P1 fixed): with g_i = dkl[b,h,i],
 *   dS2 = g_i * (P2 - P1),  dQ2 = scale2 * dS2 K2,  dK2 = scale2 * dS2^T Q2,
 * where P_k = exp(S_k - LSE_k) is rebuilt tile by tile from lse1 and lse2
 * as written by skl_forward (article section "Backward: recompute-based
 * tile-by-tile gradients"), with the kernels of `algo` (skl_bwd_algo).
 * dq2 and dk2 have the element type of the inputs and the same strides as
 * q2 and k2 respectively.  ws: skl_backward_workspace_size(shape, 0, algo)
 * bytes, 16-byte aligned, owned by the caller and overwritten by the call.
 * It may be NULL when that size is 0; for SKL_BWD_SPLIT it may be NULL (or
 * smaller) in any case, and the dQ kernel then runs over all keys unsplit.
 */
skl_status skl_backward_student(const skl_shape* shape,
                                const void* q1, const void* k1, const void* q2, const void* k2,
                                float scale1, float scale2, int causal,
                                const float* lse1, const float* lse2, const float* dkl,
                                void* dq2, void* dk2, int algo, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * Backward, "optimise P1" (the teacher, P2 fixed):
 *   r_ij = (S1 - LSE1) - (S2 - LSE2)     (log P1 - log P2 from the logits),
 *   dS1 = g_i * P1 * (r - kl_i),  dQ1 = scale1 * dS1 K1,  dK1 = scale1 * dS1^T Q1.
 * The log-ratio is never formed from log P, so probabilities that underflow
 * give exact zeros instead of NaN (article section "Backward:
 * recompute-based tile-by-tile gradients").  kl is the forward's output.
 * dq1/dk1 have the strides of q1/k1.  algo and ws as for the student, with
 * skl_backward_workspace_size(shape, 1, algo).
 */
skl_status skl_backward_teacher(const skl_shape* shape,
                                const void* q1, const void* k1, const void* q2, const void* k2,
                                float scale1, float scale2, int causal,
                                const float* lse1, const float* lse2, const float* kl,
                                const float* dkl, void* dq1, void* dk1, int algo, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/*
 * Both settings in one pass: (dq1, dk1) as skl_backward_teacher and
 * (dq2, dk2) as skl_backward_student would write them, from one recompute of
 * the two logit tiles and one pair of exponentials per (query, key) pair --
 * the two settings share every step up to dS (article section "Backward:
 * recompute-based tile-by-tile gradients").  With the student's and the
 * teacher's calls together this is the gradient of sum_i dkl_i KL_i with
 * respect to all four inputs.  Kernels: a joint dK kernel and a joint dQ
 * kernel (no atomics, bitwise deterministic); when both settings need
 * gradients this is the faster route (on MI355X about 0.8x the time of the
 * student and teacher calls at 64K tokens).  ws is optional:
 * skl_backward_joint_workspace_size(shape) is nonzero only when the query
 * tiles alone cannot fill the device, and given that many bytes (16-byte
 * aligned) the call runs the two SKL_BWD_SPLIT settings one after the other
 * instead, each with its dQ over key ranges (the student's workspace first,
 * then the teacher's); with ws NULL it always runs the joint kernels.  Outputs
 * have the dtype of the inputs and the strides of q1, k1, q2, k2.  Event
 * slots (skl_set_kernel_events): 0 before, 1 after the joint dK kernel, 2
 * after the joint dQ kernel.
 */
size_t skl_backward_joint_workspace_size(const skl_shape* shape);
skl_status skl_backward_joint(const skl_shape* shape,
                              const void* q1, const void* k1, const void* q2, const void* k2,
                              float scale1, float scale2, int causal,
                              const float* lse1, const float* lse2, const float* kl, const float* dkl,
                              void* dq1, void* dk1, void* dq2, void* dk2,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Split count that fills a GPU with `num_cus` compute units for this shape
 * (1 when the query tiles alone fill it).  Pure host arithmetic.
 */
int skl_recommended_splits(const skl_shape* shape, int causal, int num_cus);

/*
 * Profiling aid.  After this call, every entry point called on this thread
 * records events[0] on its stream right before enqueueing its first main
 * kernel and events[k] right after its k-th main kernel (k < count), so
 * hipEventElapsedTime(events[k-1], events[k]) is the k-th kernel's duration.
 * Main kernels: the forward or split-K forward kernel's main pass (one; its
 * fixup pass, which recomputes only the tiles the main pass marked, is not
 * counted); the split backward's dK kernel then dQ kernel (two); the fused
 * backward kernel (one).  Workspace clears, the reduce and the dQ convert are
 * not counted.
 * count = 0 switches it off; at most 4 events.  The events stay owned by the
 * caller.
 */
skl_status skl_set_kernel_events(hipEvent_t* events, int count);

/* Static description of a status code. */
const char* skl_status_string(skl_status status);

/* Message of the last failing call on this thread ("" if none). */
const char* skl_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int skl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STREAMKL_H */
