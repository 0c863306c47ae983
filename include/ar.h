/*
 * ar.h - C ABI of the MI355X (gfx950) all-reduce core.
 *
 * One GPU's share of a tensor-parallel all-reduce: the R rank-partial
 * activation buffers that a row-parallel linear produces, all resident in this
 * GPU's HBM, are summed elementwise, either alone (fusion op NONE) or fused
 * with the GEMM bias add, the residual add and RMSNorm over each row of
 * hidden_size elements (fusion op RESIDUAL_RMS_NORM).
 *
 * Sources:
 *   - "All Reduce Plugin" (TensorRT-Edge-LLM C++ API), class AllReducePlugin:
 *     the op is a SUM over tensor-parallel ranks of the activations after a
 *     row-parallel linear; with one rank it is a passthrough. Its enqueue()
 *     takes the caller's stream and returns an int32 status without throwing;
 *     the same convention is used here.
 *   - "type.d2", class AllReduceParams (elts_total, the per-rank buffer
 *     array bounded by MAX_RANKS_PER_NODE, local_output_buffer_ptr,
 *     fusion_params) and class AllReduceFusionParams (bias_buffer - the GEMM
 *     bias -, residual_buffer, hidden_size, weight_buffer, eps,
 *     intermediate_buffer); enum AllReduceFusionOp {NONE = 0,
 *     RESIDUAL_RMS_NORM = 1}.
 *   - "allreduce.d2", kernels customAllReduceKernels.cu: the host dispatch
 *     customAllReduce -> configurationSupported / AllReduceDispatchType ->
 *     ...RanksPerNode -> standalone (oneShotAllReduceKernel) or fused
 *     (one_shot_all_reduce_norm_kernel -> rms_norm).
 *
 * What each call computes (fp32 arithmetic inside, one rounding to the
 * element type T with round-to-nearest-even for every stored value):
 *   ar_sum:               out[i] = T( P0[i] + P1[i] + ... + P(R-1)[i] )
 *                         added left to right in rank order, starting from P0.
 *   ar_residual_rmsnorm:  a = ((P0[i] + ... + P(R-1)[i]) + bias[h]) + residual[i]
 *                         S[i] = T(a)                     -> intermediate_buffer
 *                         out[i] = T( S[i] * rstd(t) * weight[h] ),
 *                         rstd(t) = 1 / sqrt( sum_h S[t,h]^2 / hidden_size + eps )
 *                         for row t = i / hidden_size, column h = i % hidden_size.
 *
 * Device: every buffer of a call must be on the calling thread's current HIP
 * device, where the kernels are launched (the stream must belong to it too).
 *
 * Layout: every full-size buffer is a dense row-major [elts_total / H, H]
 * array of T (for ar_sum, simply elts_total contiguous elements); bias and
 * weight are [H]. All element types alike: inputs, outputs, bias, residual,
 * weight and intermediate share the one dtype.
 *
 * Ownership and execution: the caller owns every buffer (device memory, e.g.
 * from torch). The library allocates no device memory, keeps no state between
 * calls that affects results (it caches each device's CU count and kernel
 * occupancies, by device index) and needs no workspace. Calls are
 * asynchronous on the caller's HIP stream (NULL = the default stream):
 * outputs are valid once the stream has been synchronized. Calls are
 * re-entrant and thread-safe.
 *
 * Errors: every entry point returns AR_OK (0) or a negative AR_ERR_* code and
 * never throws. On a validation error nothing is launched and no output is
 * touched. Validation makes no HIP call, so it works on a host without a GPU.
 *
 * Diagnostics: with the environment variable AR_LOG set to anything but
 * "0" when the library is first used (it is read once per process), every
 * launch prints its dispatch decision to stderr - kernel, rank count, shape,
 * grid and workgroup size - and a failed launch prints the HIP error text.
 * Validation errors print nothing; they are returned as status codes.
 *
 * Size bound: elts_total * sizeof(T) must fit in size_t, and every buffer's
 * byte range [ptr, ptr + bytes) (full-size buffers: elts_total elements;
 * bias and weight: hidden_size elements) must end inside the address space.
 * A call that breaks either is AR_ERR_SHAPE (no such buffer can exist), so
 * no size check or aliasing check ever works on a wrapped byte count.
 */
#ifndef TENSOR_ALL_REDUCE_AR_H
#define TENSOR_ALL_REDUCE_AR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Upper bound on the rank count: tensor-parallel sizes 1..8 on one node
 * (MAX_RANKS_PER_NODE of "type.d2" AllReduceParams; the page leaves its value
 * unprinted). */
#define AR_MAX_RANKS 8

/* Element type of every buffer of one call. fp16 is IEEE binary16; bf16 is the
 * upper half of an IEEE binary32. */
typedef enum { AR_FP32 = 0, AR_FP16 = 1, AR_BF16 = 2 } ar_dtype_t;

/* "type.d2" enum AllReduceFusionOp, same values. The op is chosen by which
 * entry point is called; the enum is used by ar_configuration_supported. */
typedef enum { AR_FUSION_NONE = 0, AR_FUSION_RESIDUAL_RMS_NORM = 1 } ar_fusion_op_t;

/* Status codes. */
enum {
    AR_OK = 0,
    AR_ERR_NULL = -1,   /* a required pointer is NULL                              */
    AR_ERR_RANKS = -2,  /* ranks outside 1..AR_MAX_RANKS                           */
    AR_ERR_DTYPE = -3,  /* dtype is not an ar_dtype_t                              */
    AR_ERR_SHAPE = -4,  /* hidden_size <= 0, elts_total % hidden_size != 0, or a
                           buffer size past the size bound above (or an unknown
                           fusion op where one is asked for)                      */
    AR_ERR_EPS = -5,    /* eps is NaN, infinite or negative                        */
    AR_ERR_ALIAS = -6,  /* an output partly overlaps an input or the other output  */
    AR_ERR_ALIGN = -7,  /* a buffer is not aligned to the element size             */
    AR_ERR_SLICE = -8,  /* slice index or slice count out of range                 */
    AR_ERR_HIP = -100   /* a HIP launch or copy failed; see ar_last_hip_error()    */
};

/* Mirrors "type.d2" AllReduceFusionParams, field for field. Read by the fused
 * entry points (ar_residual_rmsnorm, ar_rmsnorm, ar_residual_rmsnorm_slice). */
typedef struct {
    const void *bias_buffer;     /* [H] of T: the GEMM bias, added once per
                                    element after the rank sum. NULL = no bias. */
    const void *residual_buffer; /* [elts_total] of T, added after the bias.
                                    NULL = no residual.                        */
    int32_t hidden_size;         /* H > 0, the RMSNorm width; elts_total % H == 0 */
    const void *weight_buffer;   /* [H] of T: RMSNorm scale. Required.         */
    float eps;                   /* >= 0 and finite; added to the mean square
                                    inside the square root.                    */
    void *intermediate_buffer;   /* [elts_total] of T, OUTPUT: the pre-norm sum S.
                                    Required. May be the residual buffer itself
                                    (then S replaces the residual in place).    */
} ar_fusion_params_t;

/* Mirrors "type.d2" AllReduceParams. elts_per_rank / elts_per_block are
 * derived inside the library; local_rank and local_input_buffer_ptr have no
 * meaning when all R partials are local and of equal standing. */
typedef struct {
    size_t elts_total;                           /* elements per partial; 0 = no-op   */
    int32_t ranks;                               /* R, 1..AR_MAX_RANKS                 */
    int32_t dtype;                               /* an ar_dtype_t                      */
    const void *input_buffer_ptrs[AR_MAX_RANKS]; /* R partials of [elts_total] T, in
                                                    rank order; entries >= R ignored   */
    void *local_output_buffer_ptr;               /* [elts_total] of T, OUTPUT. May be
                                                    one of the partials (in place).    */
    ar_fusion_params_t fusion_params;            /* read by the fused entry points     */
} ar_params_t;

/*
 * Fusion op NONE: out = sum of the R partials (standalone branch of
 * "allreduce.d2"; the sum of "All Reduce Plugin"). With R = 1 this is a
 * bit-exact passthrough: nothing runs when the output is the input, otherwise
 * a device-to-device copy. elts_total may be any size (no multiple of 16 bytes
 * needed) and pointers need only element alignment; 16-byte aligned pointers
 * take the vector path. fusion_params is ignored.
 * Aliasing: the output may equal a partial exactly; partial overlap is
 * AR_ERR_ALIAS.
 */
int32_t ar_sum(const ar_params_t *p, void *hip_stream);

/*
 * Fusion op RESIDUAL_RMS_NORM: pre-norm sum S to intermediate_buffer and the
 * normed output to local_output_buffer_ptr (fused branch of "allreduce.d2",
 * one_shot_all_reduce_norm_kernel -> rms_norm, with the fields of "type.d2"
 * AllReduceFusionParams). R = 1 still applies bias, residual and the norm.
 * Aliasing: the output and the intermediate may each equal a partial, and the
 * intermediate may equal the residual; outputs may not overlap each other,
 * bias or weight, and no partial overlap is allowed (AR_ERR_ALIAS).
 * Rows of more than 4096 16-byte packs (hidden > 32768 in fp16/bf16, > 16384
 * in fp32) run as three kernels on the stream, which pass each row's partial
 * sums of squares through the first 4 bytes of every 1024-pack chunk of the
 * output before writing the final values there; the output is meaningful,
 * as always, only once the call's work on the stream has completed.
 */
int32_t ar_residual_rmsnorm(const ar_params_t *p, void *hip_stream);

/*
 * The unfused branch's norm step ("allreduce.d2": after the two-shot
 * all-reduce, rms_norm_kernel_launcher -> rms_norm_kernel): the same op as
 * ar_residual_rmsnorm with a single input, x = input_buffer_ptrs[0]:
 * intermediate = T((x + bias) + residual), out = RMSNorm(intermediate) * weight.
 * Together with ar_sum it forms the unfused path (sum to a buffer, then norm),
 * the baseline that shows what fusion saves. Requires ranks == 1
 * (AR_ERR_RANKS otherwise); other rules as ar_residual_rmsnorm.
 */
int32_t ar_rmsnorm(const ar_params_t *p, void *hip_stream);

/*
 * Two-shot work split on one GPU: the share of slice `slice` (0-based) of
 * `num_slices` (1..1024; a two-shot all-reduce over R ranks uses R slices,
 * "allreduce.d2" twoShotAllReduceKernel, "type.d2" elts_per_rank). The slice
 * is written in place into the full output buffers, so running every slice
 * leaves exactly the result of the unsliced call (the all-gather layout).
 *   ar_sum_slice:              elements [begin, end) of ar_sum; slices are
 *                              equal shares of ceil(N / S) elements rounded up
 *                              to whole 16-byte packs (the last may be short
 *                              or empty).
 *   ar_residual_rmsnorm_slice: whole rows: equal shares of ceil(rows / S) rows.
 * p describes the FULL buffers and is validated as for the unsliced call.
 * A slice that is empty returns AR_OK without launching anything. Bad slice
 * arguments return AR_ERR_SLICE.
 */
int32_t ar_sum_slice(const ar_params_t *p, int32_t slice, int32_t num_slices, void *hip_stream);
int32_t ar_residual_rmsnorm_slice(const ar_params_t *p, int32_t slice, int32_t num_slices, void *hip_stream);

/* Element range [*begin, *end) that the slice call above covers, for the
 * given fusion op (an ar_fusion_op_t). Validates p like the matching call;
 * makes no HIP call. */
int32_t ar_slice_range(const ar_params_t *p, int32_t fusion_op, int32_t slice, int32_t num_slices, size_t *begin,
                       size_t *end);

/*
 * "allreduce.d2" configurationSupported: validates p for the given fusion op
 * (an ar_fusion_op_t) without launching anything. Returns 1 when the call
 * takes the 16-byte vector path, 0 when it is valid but takes the general
 * (element-wise) path, or a negative AR_ERR_* code when it is invalid.
 */
int32_t ar_configuration_supported(const ar_params_t *p, int32_t fusion_op);

/* Scratch bytes a call needs from the caller: always 0 (cf. the plugin's
 * getWorkspaceSize on the "All Reduce Plugin" page). p may be NULL. */
size_t ar_workspace_size(const ar_params_t *p);

/* Byte distance added between consecutive partial slots by ar_partials_layout,
 * and the alignment of every slot. */
#define AR_SLOT_STAGGER_BYTES 4096
#define AR_SLOT_ALIGN_BYTES 256

/*
 * Layout of the R partials in one caller-owned allocation (the one-GPU
 * counterpart of the comm-buffer workspace that CustomAllReduceHelper sizes
 * and allocates in "allreduce.d2"). Slot r starts at
 *     slot_offsets[r] = r * (round_up(elts_total * sizeof(T), AR_SLOT_ALIGN_BYTES)
 *                            + AR_SLOT_STAGGER_BYTES)
 * bytes from the base, and *total_bytes is the size to allocate (R slots).
 * Separate allocations of a large power-of-two size place element i of every
 * partial at the same offset within the same HBM interleave pattern; the
 * stagger moves each partial by 4 KiB more than the previous one, which the
 * fused kernel reads faster (about 5 % on MI355X at 8 bf16 partials of
 * [2048, 8192]). Any layout stays valid for every entry point; this one is a
 * recommendation. The base must be AR_SLOT_ALIGN_BYTES-aligned (hipMalloc and
 * torch allocations are) so that every slot takes the 16-byte vector path.
 * slot_offsets has room for `ranks` entries. Makes no HIP call.
 * Returns AR_OK, AR_ERR_RANKS, AR_ERR_DTYPE, AR_ERR_NULL, or AR_ERR_SHAPE when
 * the allocation's size (ranks slots) would not fit size_t; on an error the
 * outputs are untouched.
 */
int32_t ar_partials_layout(size_t elts_total, int32_t dtype, int32_t ranks, size_t *slot_offsets,
                           size_t *total_bytes);

/* Static, never-NULL description of a status code (unknown codes included).
 * Errors cross this boundary as int32 status codes, never as exceptions, as in
 * the plugin's enqueue() on the "All Reduce Plugin" page (declared noexcept,
 * returning int32_t); this call turns a code into text for the caller's log. */
const char *ar_status_string(int32_t status);

/* The hipError_t (as int) of the last failed HIP call made by this library on
 * the calling thread, or 0 if none failed. Not reset by later successes. The
 * detail behind AR_ERR_HIP, which keeps the int32-status convention of the
 * plugin's enqueue() ("All Reduce Plugin") while still naming the runtime's
 * own error. */
int32_t ar_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TENSOR_ALL_REDUCE_AR_H */
