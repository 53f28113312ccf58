// Host-side launch interface of the MSDeformAttn kernels, shared by the
// C-ABI translation unit and the translation units that instantiate the
// kernels (one per dtype, compiled in parallel): launch helpers, stage
// events, counting plan, and the per-dtype launch functions.  Internal to
// the library.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "msda.h"
#include "msda_backward.hpp"
#include "msda_forward.hpp"
#include "msda_plan.hpp"

namespace msda_host {

using msda::kBF16;
using msda::kBlock;
using msda::kF16;
using msda::kF32;

using msda_plan::LaneSplit;

#define MSDA_TRY(expr)                                  \
    do {                                                \
        msda_status_t s_ = (expr);                      \
        if (s_ != MSDA_SUCCESS) return s_;              \
    } while (0)

// Launch through hipLaunchKernel, whose return code belongs to this launch
// alone (no sticky error of an earlier, unrelated call is read or cleared).
template <typename... Args>
msda_status_t launch(const void* kernel, int64_t blocks, int threads, size_t lds_bytes, hipStream_t stream,
                     Args... args) {
    if (blocks <= 0) return MSDA_SUCCESS;
    if (blocks > 0x7fffffff) return MSDA_ERROR_NOT_SUPPORTED;
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), argv, lds_bytes,
                           stream) == hipSuccess
               ? MSDA_SUCCESS
               : MSDA_ERROR_HIP;
}

template <typename K>
const void* kfn(K* k) { return reinterpret_cast<const void*>(k); }

using msda_plan::count_chunk;
using msda_plan::count_chunks;
using msda_plan::fused_count_scan;

// Records events[k] (when events is not NULL) on the stream just before
// backward stage k; stage kStageEnd marks the end of the last stage.
enum Stage { kStageZero = 0, kStageCount, kStageScan, kStageGrad, kStageAccum, kStageNarrow, kStageEnd };

inline msda_status_t mark(hipEvent_t* events, int stage, hipStream_t st) {
    if (events == nullptr) return MSDA_SUCCESS;
    return hipEventRecord(events[stage], st) == hipSuccess ? MSDA_SUCCESS : MSDA_ERROR_HIP;
}

// The launches of one dtype.  Declared here; defined in
// msda_launch_impl.hpp and instantiated once per dtype, each in a
// translation unit of its own (msda_kernels_<dtype>.hip), so that the C-ABI
// translation unit compiles no kernel.
template <int DT>
struct Launch {
    static msda_status_t forward(const LaneSplit& s, const msda::Problem& pb, int ref_dims, const void* v,
                                 const void* ref, const uint8_t* kmask, const void* loc, const void* w, void* out,
                                 int32_t* counts, int nchunks, hipStream_t st);
    static msda_status_t gradient(const LaneSplit& s, const msda::Problem& pb, bool binned, int ref_dims,
                                  const void* v, const void* ref, const uint8_t* kmask, const void* loc,
                                  const void* w, const void* gout, float* gacc, uint3* recs, int32_t* cursor,
                                  int32_t* nunits, const int32_t* multi, void* gloc, void* gw, hipStream_t st);
    static msda_status_t accumulate(const LaneSplit& s, const msda::Problem& pb, int64_t max_units, int plane_units,
                                    const void* gout, const uint3* recs, const int32_t* nunits, const int4* units,
                                    const uint8_t* kmask, float* gacc, void* gfinal, hipStream_t st);
    static msda_status_t count_scan(const msda::Problem& pb, int ref_dims, const void* ref, const void* loc,
                                    int32_t* counts, int32_t* cursor, int32_t* nunits, int32_t* multi, int4* units,
                                    int accumulate, int plane_recs, int plane_us, bool counted, hipEvent_t* ev,
                                    hipStream_t st);
};

extern template struct Launch<kF32>;
extern template struct Launch<kF16>;
extern template struct Launch<kBF16>;
extern template struct Launch<msda::kF16M>;
extern template struct Launch<msda::kBF16M>;

}  // namespace msda_host
