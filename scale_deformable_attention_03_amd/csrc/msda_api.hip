// C ABI of the MSDeformAttn core (declarations and contract: include/msda.h).
//
// Host side only: validate the descriptor, plan the launch (level table,
// key segments of the binned backward, workspace layout), choose the kernel
// instantiations, enqueue.  No allocation, no host synchronisation, no state
// between calls.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "msda.h"
#include "msda_launch.hpp"

namespace {

using msda::kBF16;
using msda::kBlock;
using msda::kF16;
using msda::kF32;
using msda_host::kfn;
using msda_plan::BackwardPlan;
using msda_plan::check_problem;
using msda_plan::count_chunks;
using msda_plan::elem_bytes;
using msda_plan::fill_blocks;
using msda_plan::fused_count_scan;
using msda_plan::lane_split;
using msda_plan::LaneSplit;
using msda_plan::Layout;
using msda_plan::layout;
using msda_plan::out_elems;
using msda_plan::pack;
using msda_plan::plan_backward;
using msda_plan::plane_records;
using msda_plan::plane_units;
using msda_plan::sample_elems;
using msda_plan::value_dtype;
using msda_plan::value_elems;
using msda_host::launch;
using msda_host::Launch;
using msda_host::mark;
using msda_host::kStageZero;
using msda_host::kStageCount;
using msda_host::kStageScan;
using msda_host::kStageGrad;
using msda_host::kStageAccum;
using msda_host::kStageNarrow;
using msda_host::kStageEnd;

// Calls f(std::integral_constant<int, code>) for the kernels' dtype code.
template <typename F>
msda_status_t by_code(msda_dtype_t dt, F&& f) {
    switch (dt) {
        case MSDA_F32: return f(std::integral_constant<int, kF32>{});
        case MSDA_F16: return f(std::integral_constant<int, kF16>{});
        case MSDA_BF16: return f(std::integral_constant<int, kBF16>{});
        case MSDA_F16_F32: return f(std::integral_constant<int, msda::kF16M>{});
        default: return f(std::integral_constant<int, msda::kBF16M>{});
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A device pointer must be non-NULL when its tensor has elements, and
// 16-byte aligned when non-NULL.
msda_status_t check_ptr(const void* ptr, int64_t elems) {
    if (elems > 0 && ptr == nullptr) return MSDA_ERROR_INVALID_VALUE;
    if (ptr != nullptr && !aligned16(ptr)) return MSDA_ERROR_MISALIGNED;
    return MSDA_SUCCESS;
}

msda_status_t zero_bytes(void* p, size_t bytes, hipStream_t st) {
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    return launch(kfn(&msda::msda_zero_kernel), fill_blocks(n16), kBlock, 0, st, static_cast<uint4*>(p), n16);
}

// Reference points of the fused prologue: ref_dims 0 (none; ref unused), 2
// or 4, with [batch, num_queries, num_levels, ref_dims] elements.
msda_status_t check_ref(const msda_problem_t* p, int ref_dims, const void* ref) {
    if (ref_dims == 0) return MSDA_SUCCESS;
    if (ref_dims != 2 && ref_dims != 4) return MSDA_ERROR_INVALID_VALUE;
    return check_ptr(ref, int64_t(p->batch) * p->num_queries * p->num_levels * ref_dims);
}

// Whether a counting forward fills the backward's histogram rows: binned
// problems with samples whose planes are counted apart from the scan (small
// planes count and scan in one launch inside the backward).
bool forward_counts(const msda_problem_t* problem, const msda::Problem& pb) {
    return sample_elems(problem) > 0 && value_elems(problem) > 0 && layout(problem, pb).binned &&
           !fused_count_scan(pb);
}

// The forward.  ws != null (plain form only): also count the backward's
// records into the workspace's histogram rows (zeroed first), for a
// following msda_backward_counted on the same workspace.
msda_status_t forward_call(const msda_problem_t* problem, int ref_dims, const void* value, const void* ref,
                           const uint8_t* kmask, const void* sampling_locations, const void* attention_weights,
                           void* output, char* ws, hipStream_t stream) {
    MSDA_TRY(check_problem(problem));
    MSDA_TRY(check_ref(problem, ref_dims, ref));
    MSDA_TRY(check_ptr(value, value_elems(problem)));
    MSDA_TRY(check_ptr(sampling_locations, sample_elems(problem)));
    MSDA_TRY(check_ptr(attention_weights, sample_elems(problem)));
    MSDA_TRY(check_ptr(output, out_elems(problem)));
    if (out_elems(problem) == 0) return MSDA_SUCCESS;
    const msda::Problem pb = pack(problem);
    const LaneSplit s = lane_split(problem->embed_dims, problem->dtype);
    int32_t* counts = nullptr;
    int nchunks = 0;
    if (ws != nullptr && ref_dims == 0 && forward_counts(problem, pb)) {
        const Layout lay = layout(problem, pb);
        counts = reinterpret_cast<int32_t*>(ws + lay.counts);
        nchunks = msda::kForwardCountRows;
        // (the rows' region is padded to 256 bytes: zeroed whole, in 16-byte words)
        MSDA_TRY(zero_bytes(counts, msda_plan::round_up(size_t(pb.nplanes) * pb.nseg * nchunks * 4), stream));
    }
    return by_code(problem->dtype, [&](auto c) {
        return Launch<decltype(c)::value>::forward(s, pb, ref_dims, value, ref, kmask, sampling_locations,
                                                   attention_weights, output, counts, nchunks, stream);
    });
}

msda_status_t check_backward_ptrs(const msda_problem_t* problem, const void* value,
                                  const void* sampling_locations, const void* attention_weights,
                                  const void* grad_output, const void* grad_value,
                                  const void* grad_sampling_locations,
                                  const void* grad_attention_weights) {
    const int64_t nv = value_elems(problem), ns = sample_elems(problem), no = out_elems(problem);
    MSDA_TRY(check_ptr(value, nv));
    MSDA_TRY(check_ptr(sampling_locations, ns));
    MSDA_TRY(check_ptr(attention_weights, ns));
    MSDA_TRY(check_ptr(grad_output, no));
    MSDA_TRY(check_ptr(grad_value, nv));
    MSDA_TRY(check_ptr(grad_sampling_locations, ns));
    MSDA_TRY(check_ptr(grad_attention_weights, ns));
    return MSDA_SUCCESS;
}


// Dtype dispatch of the backward's launches.
msda_status_t gradient(msda_dtype_t dt, const LaneSplit& s, const msda::Problem& pb, bool binned, int ref_dims,
                       const void* v, const void* ref, const uint8_t* kmask, const void* loc, const void* w,
                       const void* gout, float* gacc, uint3* recs, int32_t* cursor, int32_t* nunits,
                       const int32_t* multi, void* gloc, void* gw, hipStream_t st) {
    return by_code(dt, [&](auto c) {
        return Launch<decltype(c)::value>::gradient(s, pb, binned, ref_dims, v, ref, kmask, loc, w, gout, gacc, recs,
                                                    cursor, nunits, multi, gloc, gw, st);
    });
}

msda_status_t accumulate_rows(msda_dtype_t dt, const LaneSplit& s, const msda::Problem& pb, int64_t max_units,
                              int plane_units, const void* gout, const uint3* recs, const int32_t* nunits,
                              const int4* units, const uint8_t* kmask, float* gacc, void* gfinal, hipStream_t st) {
    return by_code(dt, [&](auto c) {
        return Launch<decltype(c)::value>::accumulate(s, pb, max_units, plane_units, gout, recs, nunits, units,
                                                      kmask, gacc, gfinal, st);
    });
}

msda_status_t count_scan(msda_dtype_t dt, const msda::Problem& pb, int ref_dims, const void* ref,
                         const void* loc, int32_t* counts, int32_t* cursor, int32_t* nunits, int32_t* multi,
                         int4* units, int accumulate, int plane_recs, int plane_us, bool counted, hipEvent_t* ev,
                         hipStream_t st) {
    return by_code(dt, [&](auto c) {
        return Launch<decltype(c)::value>::count_scan(pb, ref_dims, ref, loc, counts, cursor, nunits, multi, units,
                                                      accumulate, plane_recs, plane_us, counted, ev, st);
    });
}

// The backward.  accumulate = 1: grad_value is added into the float32
// buffer gacc (gfinal unused).  accumulate = 0: grad_value is overwritten
// into gfinal, the caller's tensor of the problem's dtype; gacc is gfinal for
// float32 and the workspace's float32 buffer for 16-bit dtypes, which then
// holds only rows the kernels add into (and is rounded into gfinal at the
// end).
// ref_dims != 0: the fused prologue (loc and w are the offsets and logits,
// gloc and gw receive their gradients).  counted: a counting forward on the
// same locations filled the histogram rows (see forward_counts).
msda_status_t backward_into(const msda_problem_t* problem, int ref_dims, const void* value, const void* ref,
                            const uint8_t* kmask, const void* loc, const void* w, const void* gout, float* gacc,
                            void* gfinal, void* gloc, void* gw, char* ws, int accumulate, bool counted,
                            hipEvent_t* ev, hipStream_t st) {
    // which launches run, and their grids, come from the host plan (checked
    // on the CPU in the tests)
    const BackwardPlan plan = plan_backward(problem, accumulate != 0);
    if (sample_elems(problem) == 0) {
        // no samples (Q = 0): grad_value is zero and nothing else is written
        MSDA_TRY(mark(ev, kStageZero, st));
        if (plan.zero_blocks > 0)
            MSDA_TRY(zero_bytes(gfinal, size_t(value_elems(problem)) * (problem->dtype == MSDA_F32 ? 4 : 2), st));
        for (int stage = kStageCount; stage <= kStageNarrow; ++stage) MSDA_TRY(mark(ev, stage, st));
        return MSDA_SUCCESS;
    }
    const msda::Problem pb = pack(problem);
    const Layout lay = layout(problem, pb);
    const LaneSplit s = lane_split(problem->embed_dims, problem->dtype);
    if (!plan.binned) {
        // Float atomics straight into gacc.
        MSDA_TRY(mark(ev, kStageZero, st));
        if (plan.zero_blocks > 0) MSDA_TRY(zero_bytes(gacc, size_t(value_elems(problem)) * 4, st));
        MSDA_TRY(mark(ev, kStageCount, st));
        MSDA_TRY(mark(ev, kStageScan, st));
        MSDA_TRY(mark(ev, kStageGrad, st));
        MSDA_TRY(gradient(problem->dtype, s, pb, false, ref_dims, value, ref, kmask, loc, w, gout, gacc,
                          static_cast<uint3*>(nullptr), static_cast<int32_t*>(nullptr), static_cast<int32_t*>(nullptr),
                          static_cast<const int32_t*>(nullptr), gloc, gw, st));
        MSDA_TRY(mark(ev, kStageAccum, st));
        MSDA_TRY(mark(ev, kStageNarrow, st));
        if (plan.narrow_blocks > 0) {
            const int64_t n8 = value_elems(problem) / 8;
            const void* k = value_dtype(problem->dtype) == MSDA_F16 ? kfn(&msda::msda_narrow_kernel<kF16>)
                                                                    : kfn(&msda::msda_narrow_kernel<kBF16>);
            MSDA_TRY(launch(k, plan.narrow_blocks, kBlock, 0, st, reinterpret_cast<const float4*>(gacc),
                            static_cast<uint4*>(gfinal), n8));
        }
        return MSDA_SUCCESS;
    }
    // the accumulation reads words only a gradient workgroup writes
    if (plan.accum_blocks > 0 && plan.grad_blocks < 1) return MSDA_ERROR_INVALID_VALUE;
    int32_t* counts = reinterpret_cast<int32_t*>(ws + lay.counts);
    int32_t* cursor = reinterpret_cast<int32_t*>(ws + lay.cursor);
    int32_t* nunits = reinterpret_cast<int32_t*>(ws + lay.nunits);
    int32_t* multi = reinterpret_cast<int32_t*>(ws + lay.multi);
    int4* units = reinterpret_cast<int4*>(ws + lay.units);
    uint3* recs = reinterpret_cast<uint3*>(ws + lay.recs);

    MSDA_TRY(mark(ev, kStageZero, st));             // no zero fill on this path
    const int prec = static_cast<int>(plane_records(problem)), pun = static_cast<int>(plane_units(problem, pb));
    MSDA_TRY(count_scan(problem->dtype, pb, ref_dims, ref, loc, counts, cursor, nunits, multi, units, accumulate,
                        prec, pun, counted && ref_dims == 0 && forward_counts(problem, pb), ev, st));
    MSDA_TRY(mark(ev, kStageGrad, st));
    MSDA_TRY(gradient(problem->dtype, s, pb, true, ref_dims, value, ref, kmask, loc, w, gout, gacc, recs, cursor,
                      nunits, static_cast<const int32_t*>(multi), gloc, gw, st));
    MSDA_TRY(mark(ev, kStageAccum, st));
    MSDA_TRY(accumulate_rows(problem->dtype, s, pb, plan.accum_blocks, pun, gout, static_cast<const uint3*>(recs),
                             static_cast<const int32_t*>(nunits), static_cast<const int4*>(units), kmask, gacc,
                             plan.narrow_blocks > 0 ? gfinal : nullptr, st));
    MSDA_TRY(mark(ev, kStageNarrow, st));
    if (plan.narrow_blocks > 0) {
        const void* k = value_dtype(problem->dtype) == MSDA_F16 ? kfn(&msda::msda_narrow_segments_kernel<kF16>)
                                                                : kfn(&msda::msda_narrow_segments_kernel<kBF16>);
        MSDA_TRY(launch(k, plan.narrow_blocks, kBlock, 0, st, static_cast<const float*>(gacc), gfinal,
                        static_cast<const int32_t*>(nunits), static_cast<const int32_t*>(multi), pb));
    }
    return MSDA_SUCCESS;
}

msda_status_t backward_call(const msda_problem_t* problem, int ref_dims, const void* value, const void* ref,
                            const uint8_t* kmask, const void* sampling_locations, const void* attention_weights,
                            const void* grad_output, void* grad_value, void* grad_sampling_locations,
                            void* grad_attention_weights, void* workspace, size_t workspace_bytes, hipEvent_t* ev,
                            hipStream_t stream, bool counted = false) {
    MSDA_TRY(check_problem(problem));
    MSDA_TRY(check_ref(problem, ref_dims, ref));
    MSDA_TRY(check_backward_ptrs(problem, value, sampling_locations, attention_weights, grad_output,
                                 grad_value, grad_sampling_locations, grad_attention_weights));
    const int64_t nv = value_elems(problem);
    const size_t need = nv == 0 ? 0 : layout(problem, pack(problem)).total;
    if (need > 0) {
        if (workspace_bytes < need) return MSDA_ERROR_INVALID_VALUE;
        MSDA_TRY(check_ptr(workspace, 1));
    }
    if (nv == 0) return MSDA_SUCCESS;
    char* ws = static_cast<char*>(workspace);
    const Layout lay = layout(problem, pack(problem));
    float* gacc = problem->dtype == MSDA_F32 ? static_cast<float*>(grad_value)
                                             : reinterpret_cast<float*>(ws + lay.acc);
    MSDA_TRY(backward_into(problem, ref_dims, value, ref, kmask, sampling_locations, attention_weights, grad_output,
                           gacc, grad_value, grad_sampling_locations, grad_attention_weights, ws, 0, counted, ev,
                           stream));
    return mark(ev, kStageEnd, stream);
}

// ---- scratch memory of the no-allocation backward ----------------------------
// msda_backward_noalloc takes its workspace from this file-scope array
// instead of a caller buffer.  Every GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: the array's device address on a device comes
// from hipGetSymbolAddress, taken once per device (with that device current)
// on the entry point's first call there, and only that address is ever
// passed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`.
msda_status_t scratch_for_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSDA_ERROR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MSDA_ERROR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MSDA_SUCCESS;
}

}  // namespace

extern "C" {

msda_status_t msda_validate(const msda_problem_t* problem) { return check_problem(problem); }

int32_t msda_abi_version(void) { return MSDA_ABI_VERSION; }

const char* msda_status_string(msda_status_t status) {
    switch (status) {
        case MSDA_SUCCESS: return "MSDA_SUCCESS";
        case MSDA_ERROR_INVALID_VALUE: return "MSDA_ERROR_INVALID_VALUE";
        case MSDA_ERROR_NOT_SUPPORTED: return "MSDA_ERROR_NOT_SUPPORTED";
        case MSDA_ERROR_MISALIGNED: return "MSDA_ERROR_MISALIGNED";
        case MSDA_ERROR_HIP: return "MSDA_ERROR_HIP";
        default: return "MSDA_UNKNOWN_STATUS";
    }
}

msda_status_t msda_forward(const msda_problem_t* problem, const void* value,
                           const void* sampling_locations, const void* attention_weights,
                           void* output, hipStream_t stream) {
    return forward_call(problem, 0, value, nullptr, nullptr, sampling_locations, attention_weights, output, nullptr,
                        stream);
}

msda_status_t msda_forward_train(const msda_problem_t* problem, const void* value, const void* sampling_locations,
                                 const void* attention_weights, void* output, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    MSDA_TRY(check_problem(problem));
    const size_t need = value_elems(problem) == 0 ? 0 : layout(problem, pack(problem)).total;
    if (need > 0) {
        if (workspace_bytes < need) return MSDA_ERROR_INVALID_VALUE;
        MSDA_TRY(check_ptr(workspace, 1));
    }
    return forward_call(problem, 0, value, nullptr, nullptr, sampling_locations, attention_weights, output,
                        need > 0 ? static_cast<char*>(workspace) : nullptr, stream);
}

msda_status_t msda_forward_fused(const msda_problem_t* problem, int32_t ref_dims, const void* value,
                                 const uint8_t* key_padding_mask, const void* reference_points,
                                 const void* sampling_offsets, const void* attention_logits, void* output,
                                 hipStream_t stream) {
    if (ref_dims != 2 && ref_dims != 4) return MSDA_ERROR_INVALID_VALUE;
    return forward_call(problem, ref_dims, value, reference_points, key_padding_mask, sampling_offsets,
                        attention_logits, output, nullptr, stream);
}

size_t msda_backward_workspace_bytes(const msda_problem_t* problem) {
    if (check_problem(problem) != MSDA_SUCCESS) return 0;
    if (value_elems(problem) == 0) return 0;
    return layout(problem, pack(problem)).total;
}

msda_status_t msda_backward(const msda_problem_t* problem, const void* value,
                            const void* sampling_locations, const void* attention_weights,
                            const void* grad_output, void* grad_value,
                            void* grad_sampling_locations, void* grad_attention_weights,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return backward_call(problem, 0, value, nullptr, nullptr, sampling_locations, attention_weights, grad_output,
                         grad_value, grad_sampling_locations, grad_attention_weights, workspace, workspace_bytes,
                         nullptr, stream);
}

msda_status_t msda_backward_counted(const msda_problem_t* problem, const void* value,
                                    const void* sampling_locations, const void* attention_weights,
                                    const void* grad_output, void* grad_value,
                                    void* grad_sampling_locations, void* grad_attention_weights,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return backward_call(problem, 0, value, nullptr, nullptr, sampling_locations, attention_weights, grad_output,
                         grad_value, grad_sampling_locations, grad_attention_weights, workspace, workspace_bytes,
                         nullptr, stream, true);
}

msda_status_t msda_backward_fused(const msda_problem_t* problem, int32_t ref_dims, const void* value,
                                  const uint8_t* key_padding_mask, const void* reference_points,
                                  const void* sampling_offsets, const void* attention_logits,
                                  const void* grad_output, void* grad_value, void* grad_sampling_offsets,
                                  void* grad_attention_logits, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    if (ref_dims != 2 && ref_dims != 4) return MSDA_ERROR_INVALID_VALUE;
    return backward_call(problem, ref_dims, value, reference_points, key_padding_mask, sampling_offsets,
                         attention_logits,
                         grad_output, grad_value, grad_sampling_offsets, grad_attention_logits, workspace,
                         workspace_bytes, nullptr, stream);
}

msda_status_t msda_backward_profile(const msda_problem_t* problem, const void* value,
                                    const void* sampling_locations, const void* attention_weights,
                                    const void* grad_output, void* grad_value,
                                    void* grad_sampling_locations, void* grad_attention_weights,
                                    void* workspace, size_t workspace_bytes, hipEvent_t* stage_events,
                                    hipStream_t stream) {
    if (stage_events == nullptr) return MSDA_ERROR_INVALID_VALUE;
    return backward_call(problem, 0, value, nullptr, nullptr, sampling_locations, attention_weights, grad_output,
                         grad_value, grad_sampling_locations, grad_attention_weights, workspace, workspace_bytes,
                         stage_events, stream);
}

msda_status_t msda_backward_counted_profile(const msda_problem_t* problem, const void* value,
                                            const void* sampling_locations, const void* attention_weights,
                                            const void* grad_output, void* grad_value,
                                            void* grad_sampling_locations, void* grad_attention_weights,
                                            void* workspace, size_t workspace_bytes, hipEvent_t* stage_events,
                                            hipStream_t stream) {
    if (stage_events == nullptr) return MSDA_ERROR_INVALID_VALUE;
    return backward_call(problem, 0, value, nullptr, nullptr, sampling_locations, attention_weights, grad_output,
                         grad_value, grad_sampling_locations, grad_attention_weights, workspace, workspace_bytes,
                         stage_events, stream, true);
}

msda_status_t msda_backward_accumulate(const msda_problem_t* problem, const void* value,
                                       const void* sampling_locations, const void* attention_weights,
                                       const void* grad_output, float* grad_value_acc,
                                       void* grad_sampling_locations, void* grad_attention_weights,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
    MSDA_TRY(check_problem(problem));
    MSDA_TRY(check_backward_ptrs(problem, value, sampling_locations, attention_weights, grad_output,
                                 grad_value_acc, grad_sampling_locations, grad_attention_weights));
    const size_t need = msda_backward_workspace_bytes(problem);
    if (need > 0) {
        if (workspace_bytes < need) return MSDA_ERROR_INVALID_VALUE;
        MSDA_TRY(check_ptr(workspace, 1));
    }
    if (value_elems(problem) == 0) return MSDA_SUCCESS;
    return backward_into(problem, 0, value, nullptr, nullptr, sampling_locations, attention_weights, grad_output,
                         grad_value_acc, nullptr, grad_sampling_locations, grad_attention_weights,
                         static_cast<char*>(workspace), 1, false, nullptr, stream);
}

size_t msda_backward_noalloc_max_workspace(void) { return kScratchBytes; }

msda_status_t msda_backward_noalloc(const msda_problem_t* problem, const void* value, const void* sampling_locations,
                                    const void* attention_weights, const void* grad_output, void* grad_value,
                                    void* grad_sampling_locations, void* grad_attention_weights,
                                    hipStream_t stream) {
    MSDA_TRY(check_problem(problem));
    MSDA_TRY(check_backward_ptrs(problem, value, sampling_locations, attention_weights, grad_output, grad_value,
                                 grad_sampling_locations, grad_attention_weights));
    if (value_elems(problem) == 0) return MSDA_SUCCESS;
    const size_t need = layout(problem, pack(problem)).total;
    if (need > kScratchBytes) return MSDA_ERROR_NOT_SUPPORTED;
    void* ws = nullptr;
    if (need > 0) MSDA_TRY(scratch_for_current_device(&ws));
    return backward_call(problem, 0, value, nullptr, nullptr, sampling_locations, attention_weights, grad_output,
                         grad_value, grad_sampling_locations, grad_attention_weights, ws, need, nullptr, stream);
}

}  // extern "C"
