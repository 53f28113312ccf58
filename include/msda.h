/*
 * msda.h -- C ABI of the MI355X (gfx950) multi-scale deformable attention core.
 *
 * The operation (forward):
 *   For every batch b, query q and head m, sample level l of the flattened
 *   multi-scale map bilinearly at each of its P normalised locations, weight
 *   each sample by its attention weight and sum the L*P weighted samples:
 *
 *     out[b, q, m*D + d] = sum_{l<L} sum_{p<P} w[b,q,m,l,p] *
 *                          bilinear(value_l[b, :, :, m, d], loc[b,q,m,l,p])
 *
 *   Definition: "Deformable DETR walkthrough" (zhangshiyu.com/post/59697),
 *   section 2.2.4, reference function ms_deform_attn_core_pytorch: per level,
 *   grid_sample(mode=bilinear, padding_mode=zeros, align_corners=False) at
 *   grid = 2*loc - 1, times the weights, summed over levels and points.
 *   Interface, tensor layouts and envelope: Ascend DrivingSDK API page for
 *   multi_scale_deformable_attn (prototype, parameter list, return value,
 *   constraints).  The backward returns gradients for value, locations and
 *   weights only ("DQ-DETR ops directory" CSDN page, section 2(3)).
 *
 * Conventions shared by every entry point:
 *   - Pixel coordinates: x = loc_x * W - 0.5, y = loc_y * H - 0.5, each
 *     rounded to float32 separately (no fused multiply-add).  A sample takes
 *     part only when -1 < x < W and -1 < y < H (NaN and +-Inf fail); a corner
 *     outside the map reads as zero (per-corner zero padding).
 *   - Layouts (all row-major, contiguous; float types per msda_dtype_t):
 *       value                   [batch, num_keys, num_heads, embed_dims]
 *       sampling_locations      [batch, num_queries, num_heads, num_levels, num_points, 2]  (x, y)
 *       attention_weights       [batch, num_queries, num_heads, num_levels, num_points]
 *       output / grad_output    [batch, num_queries, num_heads * embed_dims]
 *       grad_value              like value
 *       grad_sampling_locations like sampling_locations
 *       grad_attention_weights  like attention_weights
 *     Row `start_l + h*W_l + w` of value is pixel (h, w) of level l.
 *   - spatial_shapes and level_start_index are HOST arrays (int64), read
 *     during the call only; they reach the kernels as launch arguments.  The
 *     float tensors and the workspace are DEVICE pointers on the current
 *     device.
 *   - Arithmetic: inputs are widened to float32, all sums are float32, every
 *     output is rounded once (round-to-nearest-even) to the dtype.  fp16 and
 *     bf16 backward accumulate grad_value in a float32 workspace.
 *   - Ownership: the caller allocates and owns every buffer.  The library
 *     allocates nothing, keeps no state between calls, never synchronises the
 *     host, and enqueues all work on `stream` (so calls may be captured in a
 *     HIP graph).
 *   - Errors: argument problems are reported synchronously, before anything
 *     is enqueued.  A failed launch returns MSDA_ERROR_HIP.  Faults inside a
 *     kernel surface at the caller's next synchronisation, as for any HIP
 *     work.
 */
#ifndef MSDA_H_
#define MSDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSDA_ABI_VERSION 1

/* Float types of one call.  MSDA_F32, MSDA_F16, MSDA_BF16: every float
 * tensor in that type (fp32 and fp16 per the Ascend API page's dtype list;
 * bf16 in addition).  Mixed precision: MSDA_F16_F32 and MSDA_BF16_F32 keep
 * the value-side tensors (value, output, grad_output, grad_value) in fp16 /
 * bf16 and the per-sample tensors (sampling_locations, attention_weights,
 * their gradients; for the fused entry points reference_points,
 * sampling_offsets, attention_logits and their gradients) in float32, so
 * that locations and weights keep float32 resolution while the gathered
 * rows are half as wide. */
typedef enum {
    MSDA_F32 = 0,
    MSDA_F16 = 1,
    MSDA_BF16 = 2,
    MSDA_F16_F32 = 3,
    MSDA_BF16_F32 = 4
} msda_dtype_t;

typedef enum {
    MSDA_SUCCESS = 0,
    MSDA_ERROR_INVALID_VALUE = 1, /* inconsistent sizes, NULL pointers, workspace too small */
    MSDA_ERROR_NOT_SUPPORTED = 2, /* outside the envelope below */
    MSDA_ERROR_MISALIGNED = 3,    /* a device pointer is not 16-byte aligned */
    MSDA_ERROR_HIP = 4            /* a HIP launch failed */
} msda_status_t;

/*
 * Problem descriptor.
 *   batch, num_queries          >= 0 (0 makes an empty problem: nothing to
 *                                  compute; the backward still zeroes
 *                                  grad_value)
 *   num_heads                   1..8      (Ascend constraints: heads <= 8)
 *   embed_dims                  8..256, a multiple of 8 (Ascend parameter list
 *                                  and constraints)
 *   num_levels, num_points      >= 1, num_levels * num_points <= 64 (Ascend
 *                                  constraints)
 *   num_keys                    = sum_l H_l * W_l (asserted by MSDeformAttn.forward
 *                                  in the walkthrough)
 *   spatial_shapes              host int64 [num_levels][2] = (H_l, W_l), each >= 1
 *   level_start_index           host int64 [num_levels], the exclusive prefix sum
 *                                  of H_l * W_l
 *   Index range: num_keys*num_heads*embed_dims and
 *   num_queries*num_heads*num_levels*num_points*2 must stay below 2^31 (per-batch
 *   offsets are 32-bit); larger problems return MSDA_ERROR_NOT_SUPPORTED.
 */
typedef struct {
    int32_t batch;
    int32_t num_keys;
    int32_t num_heads;
    int32_t embed_dims;
    int32_t num_levels;
    int32_t num_points;
    int32_t num_queries;
    msda_dtype_t dtype;
    const int64_t *spatial_shapes;
    const int64_t *level_start_index;
} msda_problem_t;

/*
 * msda_validate: check a descriptor on the host (no HIP call, no device
 * access).  Returns MSDA_SUCCESS, MSDA_ERROR_INVALID_VALUE or
 * MSDA_ERROR_NOT_SUPPORTED.  Every other entry point runs the same checks
 * first.
 */
msda_status_t msda_validate(const msda_problem_t *problem);

/*
 * msda_forward: output = MSDeformAttn core(value, locations, weights).
 *   value, sampling_locations, attention_weights: device, read only.
 *   output: device, overwritten in full.
 *   Every pointer 16-byte aligned; a pointer may be NULL only if its tensor
 *   has no elements.  One kernel launch on `stream`.  The result is
 *   bitwise repeatable run to run.
 */
msda_status_t msda_forward(const msda_problem_t *problem,
                           const void *value,
                           const void *sampling_locations,
                           const void *attention_weights,
                           void *output,
                           hipStream_t stream);

/*
 * msda_backward_workspace_bytes: device workspace msda_backward and
 * msda_backward_accumulate need for this problem.  It holds the binned
 * transpose of the sampling pattern (per-segment histogram rows and
 * cursors, the unit list and up to four 12-byte records per sample) and,
 * when grad_value is 16-bit, a float32 grad_value accumulator
 * (batch*num_keys*num_heads*embed_dims*4 bytes).  Returns 0 for an empty
 * problem and for an invalid descriptor; the backward then reports the
 * error.
 */
size_t msda_backward_workspace_bytes(const msda_problem_t *problem);

/*
 * msda_backward: gradients of sum(grad_output * output) with respect to
 * value, sampling_locations and attention_weights.
 *   grad_value[corner row]   += w * (bilinear weight) * grad_output, summed
 *                               over every sample; rows never sampled are 0
 *   grad_attention_weights    = <grad_output, bilinear sample>
 *   grad_sampling_locations   = (W * w * <grad_output, d sample/dx>,
 *                                H * w * <grad_output, d sample/dy>)
 *   Derivatives are taken with respect to the normalised locations (hence
 *   the factors W and H); at an integer pixel coordinate the cell that floor
 *   selects is used (the right derivative).  Samples outside the map get zero
 *   gradients.
 *   All three gradients are OVERWRITTEN (not accumulated).  grad_value sums
 *   its contributions in an order set at run time (record slots taken with
 *   atomics; float32 atomics where a key segment spans several units), so
 *   its low bits may vary from run to run; the other two gradients are
 *   bitwise repeatable.
 *   workspace: device, at least msda_backward_workspace_bytes(problem) bytes
 *   (may be NULL when that is 0), 16-byte aligned, owned by the caller; its
 *   contents are scratch on entry and on exit.  Calls that overlap in time
 *   must not share a workspace.
 *   Enqueues on `stream`: a record count and a scan (one kernel when each
 *   (batch, head) has at most 8192 samples), the gradient kernel (a
 *   gather like the forward, which also writes the records), the
 *   accumulation kernel (one workgroup per unit of a key segment; rows of
 *   a segment that fits one unit are written once) and, for a 16-bit
 *   grad_value, a kernel that rounds the rows of segments split over several
 *   units.  Problems outside the record format (2^24 or more queries, a
 *   level side above 65,534, more than 2048 key segments per (batch, head),
 *   2^30 or more records) fall back to a zero fill and float atomics.
 */
msda_status_t msda_backward(const msda_problem_t *problem,
                            const void *value,
                            const void *sampling_locations,
                            const void *attention_weights,
                            const void *grad_output,
                            void *grad_value,
                            void *grad_sampling_locations,
                            void *grad_attention_weights,
                            void *workspace,
                            size_t workspace_bytes,
                            hipStream_t stream);

/*
 * msda_forward_train: msda_forward for a training step, which also does the
 * backward's first pass.  The binned backward starts by counting each
 * sample's records per key segment from the sampling locations alone
 * (histogram rows in the workspace); this forward computes every sample's
 * bilinear cell anyway ("Deformable DETR walkthrough" section 2.2.4,
 * ms_deform_attn_core_pytorch: the grid_sample of each level), so it counts
 * them there and leaves the rows in `workspace` for msda_backward_counted.
 *   Arguments as msda_forward, plus workspace / workspace_bytes as for
 *   msda_backward (the same size, msda_backward_workspace_bytes).  The output
 *   is the one msda_forward writes, bit for bit.  Enqueues a kernel that
 *   zeroes the histogram rows, then the forward, on `stream`.  Problems whose
 *   backward counts and scans in one launch (at most 8192 samples per
 *   (batch, head)) or falls back to float atomics get a plain forward; their
 *   msda_backward_counted is then msda_backward.
 *   Errors: as msda_forward, and MSDA_ERROR_INVALID_VALUE for a missing or
 *   short workspace (checked before anything is enqueued).
 */
msda_status_t msda_forward_train(const msda_problem_t *problem,
                                 const void *value,
                                 const void *sampling_locations,
                                 const void *attention_weights,
                                 void *output,
                                 void *workspace,
                                 size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * msda_backward_counted: msda_backward after msda_forward_train, without
 * the counting pass.
 *   Arguments, results and errors as msda_backward.  Precondition: a
 *   msda_forward_train with the same problem and the same
 *   sampling_locations contents was enqueued on this workspace, and nothing
 *   else used the workspace in between (the histogram rows it left are read
 *   here; with other locations the records would overflow their segments'
 *   ranges).  Same workspace ownership rules as msda_backward.
 */
msda_status_t msda_backward_counted(const msda_problem_t *problem,
                                    const void *value,
                                    const void *sampling_locations,
                                    const void *attention_weights,
                                    const void *grad_output,
                                    void *grad_value,
                                    void *grad_sampling_locations,
                                    void *grad_attention_weights,
                                    void *workspace,
                                    size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * msda_backward_accumulate: msda_backward, adding grad_value into a float32
 * buffer instead of overwriting it.
 *   grad_value_acc (device, float32, laid out like value whatever the
 *   problem's dtype) is ACCUMULATED into: grad_value_acc[corner row] +=
 *   w * (bilinear weight) * grad_output; the caller zeroes or pre-fills it.
 *   grad_sampling_locations and grad_attention_weights (per-sample type) are
 *   overwritten, as in msda_backward.  Same kernels as msda_backward except
 *   that the accumulation kernel adds its rows with float atomics (and no
 *   conversion kernel runs).  For callers that sum the value gradient of
 *   several calls into one float32 buffer.  Same workspace, checks and error
 *   codes as msda_backward.
 */
msda_status_t msda_backward_accumulate(const msda_problem_t *problem,
                                       const void *value,
                                       const void *sampling_locations,
                                       const void *attention_weights,
                                       const void *grad_output,
                                       float *grad_value_acc,
                                       void *grad_sampling_locations,
                                       void *grad_attention_weights,
                                       void *workspace,
                                       size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * msda_backward_profile: msda_backward, recording HIP events between its
 * kernels so that a caller can time each stage on the stream.
 *   stage_events: host array of MSDA_BACKWARD_STAGES + 1 events created by
 *   the caller (hipEventCreate); event k is recorded just before stage k,
 *   the last one after the final stage:
 *     0 zero fill (float-atomic fallback only)
 *     1 count records per segment    2 scan counts into ranges
 *     3 gradient kernel (gather, records)
 *     4 accumulate grad_value        5 fp16/bf16 conversion
 *   A stage with no kernel for the problem leaves its two events back to
 *   back: stage 0 on the binned path; the scan when one kernel counts and
 *   scans (planes of at most 8192 samples); the conversion for fp32; the
 *   count, scan and accumulation on the float-atomic fallback.
 *   Otherwise identical to msda_backward; stage_events must not be NULL.
 */
#define MSDA_BACKWARD_STAGES 6
msda_status_t msda_backward_profile(const msda_problem_t *problem,
                                    const void *value,
                                    const void *sampling_locations,
                                    const void *attention_weights,
                                    const void *grad_output,
                                    void *grad_value,
                                    void *grad_sampling_locations,
                                    void *grad_attention_weights,
                                    void *workspace,
                                    size_t workspace_bytes,
                                    hipEvent_t *stage_events,
                                    hipStream_t stream);

/*
 * msda_backward_counted_profile: msda_backward_counted with the stage events
 * of msda_backward_profile (measurement only).  Stage 1 (count) has no
 * kernel where msda_forward_train counted; otherwise as
 * msda_backward_profile, with msda_backward_counted's precondition.
 */
msda_status_t msda_backward_counted_profile(const msda_problem_t *problem,
                                            const void *value,
                                            const void *sampling_locations,
                                            const void *attention_weights,
                                            const void *grad_output,
                                            void *grad_value,
                                            void *grad_sampling_locations,
                                            void *grad_attention_weights,
                                            void *workspace,
                                            size_t workspace_bytes,
                                            hipEvent_t *stage_events,
                                            hipStream_t stream);

/*
 * msda_backward_noalloc: msda_backward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *   Same arguments, semantics, checks and results as msda_backward, without
 *   the workspace arguments: the workspace comes from a scratch array of
 *   msda_backward_noalloc_max_workspace() bytes (64 MiB) that the library
 *   holds in device memory, one per GPU it runs on, until the process ends.
 *   The call allocates nothing (no hipMalloc, hipFree or allocating library
 *   routine).  Its first call on a device looks up that device's copy of the
 *   array (hipGetSymbolAddress, with the device current); make that first
 *   call outside any graph capture.
 *   A problem whose msda_backward_workspace_bytes() exceeds the maximum
 *   returns MSDA_ERROR_NOT_SUPPORTED before anything is enqueued (use
 *   msda_backward with a workspace of its own).  The array keeps the last
 *   call's contents; nothing in it needs to start at zero.
 *   Calls that overlap on one GPU (on different streams, or from several
 *   host threads without ordering) share that GPU's array and race: order
 *   them on one stream.
 */
size_t msda_backward_noalloc_max_workspace(void);
msda_status_t msda_backward_noalloc(const msda_problem_t *problem,
                                    const void *value,
                                    const void *sampling_locations,
                                    const void *attention_weights,
                                    const void *grad_output,
                                    void *grad_value,
                                    void *grad_sampling_locations,
                                    void *grad_attention_weights,
                                    hipStream_t stream);

/*
 * Fused prologue: the step that feeds the core in MSDeformAttn.forward
 * ("Deformable DETR walkthrough" (zhangshiyu.com/post/59697), section 2.2.4;
 * the two reference-point forms in sections 2.4.1 and 2.4.2, step 3), done
 * inside the kernels instead of as separate passes over HBM:
 *
 *   ref_dims = 2:  loc[b,q,m,l,p] = ref[b,q,l] + off[b,q,m,l,p] / (W_l, H_l)
 *   ref_dims = 4:  loc[b,q,m,l,p] = ref[b,q,l,0:2] +
 *                                   off[b,q,m,l,p] / P * ref[b,q,l,2:4] * 0.5
 *   w[b,q,m,:,:]  = softmax of logit[b,q,m,:,:] over its L*P entries
 *
 * then the core as in msda_forward.  Each location is formed in float32
 * one operation at a time in the order written (no fused multiply-add); the
 * softmax subtracts the group's maximum, sums exp in float32 and divides.
 *   reference_points  [batch, num_queries, num_levels, ref_dims] (x, y) or
 *                     (x, y, w, h), normalised, per-sample type
 *   sampling_offsets  [batch, num_queries, num_heads, num_levels, num_points, 2]
 *                     (x, y), in pixels of the level (2-d) or in units of
 *                     P half-box sizes (4-d)
 *   attention_logits  [batch, num_queries, num_heads, num_levels, num_points]
 *   key_padding_mask  NULL (no padding) or device uint8 [batch, num_keys]:
 *                     nonzero marks a padded key, whose value row the module
 *                     fills with zeros before the core (section 2.2.4,
 *                     masked_fill), so the kernels read it as zero; no
 *                     alignment needed
 * ref_dims must be 2 or 4 (MSDA_ERROR_INVALID_VALUE otherwise).  Pointers,
 * ownership, streams and errors as for msda_forward.
 */
msda_status_t msda_forward_fused(const msda_problem_t *problem,
                                 int32_t ref_dims,
                                 const void *value,
                                 const uint8_t *key_padding_mask,
                                 const void *reference_points,
                                 const void *sampling_offsets,
                                 const void *attention_logits,
                                 void *output,
                                 hipStream_t stream);

/*
 * msda_backward_fused: gradients of sum(grad_output * output) of
 * msda_forward_fused with respect to value, sampling_offsets and
 * attention_logits (not reference_points: the pages detach refined
 * reference points before they reach the attention, section 2.4.1 step 2,
 * and the encoder's are a fixed grid).
 *   grad_value             as msda_backward
 *   grad_sampling_offsets  = grad_sampling_locations * d loc / d off, i.e.
 *                            divided by (W_l, H_l) (2-d) or multiplied by
 *                            ref_wh * 0.5 / P (4-d); zero off the map
 *   grad_attention_logits  = w * (g - sum over the group of w * g), with g
 *                            the gradient of the weights as in msda_backward
 *                            (a sample off the map has g = 0 but still
 *                            receives the second term)
 * With a key_padding_mask the rows of padded keys read as zero in every
 * gradient, and their grad_value rows are zero (the gradient of the
 * zero-fill).
 * Same workspace (msda_backward_workspace_bytes), kernels, ownership and
 * error codes as msda_backward; all three gradients are overwritten.
 */
msda_status_t msda_backward_fused(const msda_problem_t *problem,
                                  int32_t ref_dims,
                                  const void *value,
                                  const uint8_t *key_padding_mask,
                                  const void *reference_points,
                                  const void *sampling_offsets,
                                  const void *attention_logits,
                                  const void *grad_output,
                                  void *grad_value,
                                  void *grad_sampling_offsets,
                                  void *grad_attention_logits,
                                  void *workspace,
                                  size_t workspace_bytes,
                                  hipStream_t stream);

/* msda_status_string: a static, human-readable name for a status code. */
const char *msda_status_string(msda_status_t status);

/* msda_abi_version: MSDA_ABI_VERSION of the built library. */
int32_t msda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_H_ */
