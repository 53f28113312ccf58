/*
 * msda_micro.h -- measurement kernels (libmsda_micro.so), not part of the
 * MSDeformAttn computation.
 *
 * They time the two access patterns that bound the core on this GPU, with
 * no other work around them:
 *   - gather: every (query, head) group of lanes reads the corner rows of its
 *     samples, four rows per sample, one 16-byte vector per lane per row (the
 *     forward's and the gradient's corner gather; a bilinear sample reads the
 *     four value rows around its location, "Deformable DETR walkthrough"
 *     (zhangshiyu.com/post/59697), section 2.2.4, ms_deform_attn_core_pytorch
 *     via grid_sample);
 *   - scatter: the same corner rows receive one float32 atomic add per
 *     element (how a per-sample backward scatters grad_value when it adds
 *     into shared rows directly).
 *
 * Arguments:
 *   rows / dst     device buffer of nvec 16-byte vectors (float32 rows of
 *                  4 * lanes elements each).
 *   corner_vec     device uint32 [ngroups][samples * 4]: for each corner, the
 *                  index of its row's first 16-byte vector.  The caller
 *                  guarantees corner_vec[i] + lanes <= nvec for every entry;
 *                  the kernels do not check it.
 *   out            device [ngroups][lanes] 16-byte vectors (the gather's
 *                  result, written so that the loads are not dead).
 *   ngroups        groups (for the core: batch * queries * heads).
 *   samples        samples per group (levels * points), 1 .. 64.
 *   lanes          lanes per group = row bytes / 16: 2, 4, 8 or 16.
 *   with_fma       gather: 0 = loads only (the lanes xor the loaded bits),
 *                  1 = loads plus four fp32 FMAs per element and corner.
 *   lane_contiguous scatter: 1 = lane i adds elements i, i + lanes, ...
 *                  (adjacent lanes, adjacent addresses); 0 = lane i adds its
 *                  own four consecutive elements (a 16-byte lane stride).
 *   stream         HIP stream; work is enqueued only.
 * Groups map to workgroups of 256 lanes in order, blocks spread over the
 * XCDs in contiguous runs as the core's kernels do.
 * Return: 0 success; 1 invalid argument (nothing enqueued); 4 launch failure.
 */
#ifndef MSDA_MICRO_H_
#define MSDA_MICRO_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int msda_micro_gather(const void *rows, const uint32_t *corner_vec, void *out, int64_t ngroups, int samples,
                      int lanes, int with_fma, hipStream_t stream);

int msda_micro_scatter(float *dst, const uint32_t *corner_vec, int64_t ngroups, int samples, int lanes,
                       int lane_contiguous, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_MICRO_H_ */
