// C ABI of the MSDeformAttn core (declarations and contract: include/msda.h).
//
// Host side only: validate the descriptor, pack the level table into launch
// arguments, choose the kernel instantiation, enqueue.  No allocation, no
// host synchronisation, no state between calls.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "msda.h"
#include "msda_kernels.hpp"

namespace {

using msda::kBF16;
using msda::kBlock;
using msda::kF16;
using msda::kF32;

constexpr int64_t kIndexLimit = int64_t(1) << 31;

int elem_bytes(msda_dtype_t dt) { return dt == MSDA_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Lane split of one group: VECB bytes per lane, LPR lanes (a power of two,
// at least 4) of which `active` own channels.
struct LaneSplit {
    int vecb, lpr, active;
};

LaneSplit lane_split(int embed_dims, msda_dtype_t dt) {
    const int row = embed_dims * elem_bytes(dt);   // a multiple of 16 bytes
    LaneSplit s;
    s.vecb = row >= 64 ? 16 : (row % 8 == 0 && row >= 32 ? 8 : 4);
    s.active = row / s.vecb;
    s.lpr = 4;
    while (s.lpr < s.active) s.lpr *= 2;
    return s;
}

msda_status_t check_problem(const msda_problem_t* p) {
    if (p == nullptr) return MSDA_ERROR_INVALID_VALUE;
    if (p->dtype != MSDA_F32 && p->dtype != MSDA_F16 && p->dtype != MSDA_BF16)
        return MSDA_ERROR_INVALID_VALUE;
    if (p->batch < 0 || p->num_queries < 0 || p->num_keys < 1 || p->num_heads < 1 ||
        p->embed_dims < 1 || p->num_levels < 1 || p->num_points < 1)
        return MSDA_ERROR_INVALID_VALUE;
    if (p->spatial_shapes == nullptr || p->level_start_index == nullptr)
        return MSDA_ERROR_INVALID_VALUE;
    // Envelope of the Ascend API page (constraints): L*P <= 64, heads <= 8,
    // embed_dims <= 256 and a multiple of 8.
    if (p->embed_dims % 8 != 0 || p->embed_dims > 256 || p->num_heads > 8 ||
        int64_t(p->num_levels) * p->num_points > 64)
        return MSDA_ERROR_NOT_SUPPORTED;
    int64_t keys = 0;
    for (int l = 0; l < p->num_levels; ++l) {
        const int64_t H = p->spatial_shapes[2 * l], W = p->spatial_shapes[2 * l + 1];
        if (H < 1 || W < 1 || H >= kIndexLimit || W >= kIndexLimit) return MSDA_ERROR_INVALID_VALUE;
        if (p->level_start_index[l] != keys) return MSDA_ERROR_INVALID_VALUE;
        keys += H * W;
        if (keys >= kIndexLimit) return MSDA_ERROR_INVALID_VALUE;
    }
    if (keys != p->num_keys) return MSDA_ERROR_INVALID_VALUE;
    const int64_t pitch = int64_t(p->num_heads) * p->embed_dims;
    if (int64_t(p->num_keys) * pitch >= kIndexLimit) return MSDA_ERROR_NOT_SUPPORTED;
    if (int64_t(p->num_queries) * p->num_heads * p->num_levels * p->num_points * 2 >= kIndexLimit)
        return MSDA_ERROR_NOT_SUPPORTED;
    return MSDA_SUCCESS;
}

msda::Problem pack(const msda_problem_t* p) {
    msda::Problem pb;
    memset(&pb, 0, sizeof(pb));
    pb.bs = p->batch;
    pb.K = p->num_keys;
    pb.M = p->num_heads;
    pb.D = p->embed_dims;
    pb.L = p->num_levels;
    pb.P = p->num_points;
    pb.Q = p->num_queries;
    pb.lpr_active = lane_split(p->embed_dims, p->dtype).active;
    pb.ngroups = int64_t(p->batch) * p->num_queries * p->num_heads;
    for (int l = 0; l < p->num_levels; ++l) {
        pb.lv.H[l] = static_cast<int32_t>(p->spatial_shapes[2 * l]);
        pb.lv.W[l] = static_cast<int32_t>(p->spatial_shapes[2 * l + 1]);
        pb.lv.start[l] = static_cast<int32_t>(p->level_start_index[l]);
    }
    return pb;
}

int64_t value_elems(const msda_problem_t* p) {
    return int64_t(p->batch) * p->num_keys * p->num_heads * p->embed_dims;
}
int64_t sample_elems(const msda_problem_t* p) {
    return int64_t(p->batch) * p->num_queries * p->num_heads * p->num_levels * p->num_points;
}
int64_t out_elems(const msda_problem_t* p) {
    return int64_t(p->batch) * p->num_queries * p->num_heads * p->embed_dims;
}

// A device pointer must be non-NULL when its tensor has elements, and
// 16-byte aligned when non-NULL.
msda_status_t check_ptr(const void* ptr, int64_t elems) {
    if (elems > 0 && ptr == nullptr) return MSDA_ERROR_INVALID_VALUE;
    if (ptr != nullptr && !aligned16(ptr)) return MSDA_ERROR_MISALIGNED;
    return MSDA_SUCCESS;
}

#define MSDA_TRY(expr)                                  \
    do {                                                \
        msda_status_t s_ = (expr);                      \
        if (s_ != MSDA_SUCCESS) return s_;              \
    } while (0)

// Launch through hipLaunchKernel, whose return code belongs to this launch
// alone (no sticky error of an earlier, unrelated call is read or cleared).
template <typename... Args>
msda_status_t launch(const void* kernel, unsigned blocks, size_t lds_bytes, hipStream_t stream,
                     Args... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(kernel, dim3(blocks), dim3(kBlock), argv, lds_bytes, stream) == hipSuccess
               ? MSDA_SUCCESS
               : MSDA_ERROR_HIP;
}

template <typename K>
const void* kfn(K* k) { return reinterpret_cast<const void*>(k); }

// ---- kernel selection ------------------------------------------------------

struct Launch {
    unsigned blocks;
    size_t lds_bytes;
};

Launch geometry(const msda::Problem& pb, int lpr) {
    const int64_t gpb = kBlock / lpr;
    Launch g;
    g.blocks = static_cast<unsigned>((pb.ngroups + gpb - 1) / gpb);
    g.lds_bytes = sizeof(float) * msda::lds_words(static_cast<int>(gpb), pb.L * pb.P);
    return g;
}

template <int DT, int VECB, int LPR>
msda_status_t fwd_launch(const msda::Problem& pb, const void* v, const void* loc, const void* w,
                         void* out, hipStream_t st) {
    const Launch g = geometry(pb, LPR);
    const void* k = (pb.L == 4 && pb.P == 4) ? kfn(&msda::msda_forward_kernel<DT, VECB, LPR, 4, 4>)
                                             : kfn(&msda::msda_forward_kernel<DT, VECB, LPR, 0, 0>);
    return launch(k, g.blocks, g.lds_bytes, st, v, loc, w, out, pb);
}

template <int DT, int VECB, int LPR>
msda_status_t bwd_launch(const msda::Problem& pb, const void* v, const void* loc, const void* w,
                         const void* gout, float* gacc, void* gloc, void* gw, hipStream_t st) {
    const Launch g = geometry(pb, LPR);
    const void* k = (pb.L == 4 && pb.P == 4) ? kfn(&msda::msda_backward_kernel<DT, VECB, LPR, 4, 4>)
                                             : kfn(&msda::msda_backward_kernel<DT, VECB, LPR, 0, 0>);
    return launch(k, g.blocks, g.lds_bytes, st, v, loc, w, gout, gacc, gloc, gw, pb);
}

// Calls F<DT, VECB, LPR>::run(args...) for the problem's lane split.
template <int DT, template <int, int, int> class F, typename... A>
msda_status_t by_split(const LaneSplit& s, A&&... a) {
    if (s.vecb == 4) return F<DT, 4, 4>::run(a...);
    if (s.vecb == 8) {
        if (s.lpr == 4) return F<DT, 8, 4>::run(a...);
        return F<DT, 8, 8>::run(a...);
    }
    switch (s.lpr) {
        case 4: return F<DT, 16, 4>::run(a...);
        case 8: return F<DT, 16, 8>::run(a...);
        case 16: return F<DT, 16, 16>::run(a...);
        case 32: return F<DT, 16, 32>::run(a...);
        default: return F<DT, 16, 64>::run(a...);
    }
}

template <int DT, int VECB, int LPR>
struct Fwd {
    static msda_status_t run(const msda::Problem& pb, const void* v, const void* loc, const void* w,
                             void* out, hipStream_t st) {
        return fwd_launch<DT, VECB, LPR>(pb, v, loc, w, out, st);
    }
};

template <int DT, int VECB, int LPR>
struct Bwd {
    static msda_status_t run(const msda::Problem& pb, const void* v, const void* loc, const void* w,
                             const void* gout, float* gacc, void* gloc, void* gw, hipStream_t st) {
        return bwd_launch<DT, VECB, LPR>(pb, v, loc, w, gout, gacc, gloc, gw, st);
    }
};

unsigned fill_blocks(int64_t n) {
    const int64_t want = (n + kBlock - 1) / kBlock;
    return static_cast<unsigned>(want < 8192 ? (want > 0 ? want : 1) : 8192);
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
    MSDA_TRY(check_problem(problem));
    MSDA_TRY(check_ptr(value, value_elems(problem)));
    MSDA_TRY(check_ptr(sampling_locations, sample_elems(problem)));
    MSDA_TRY(check_ptr(attention_weights, sample_elems(problem)));
    MSDA_TRY(check_ptr(output, out_elems(problem)));
    if (out_elems(problem) == 0) return MSDA_SUCCESS;
    const msda::Problem pb = pack(problem);
    const LaneSplit s = lane_split(problem->embed_dims, problem->dtype);
    switch (problem->dtype) {
        case MSDA_F32:
            return by_split<kF32, Fwd>(s, pb, value, sampling_locations, attention_weights, output, stream);
        case MSDA_F16:
            return by_split<kF16, Fwd>(s, pb, value, sampling_locations, attention_weights, output, stream);
        default:
            return by_split<kBF16, Fwd>(s, pb, value, sampling_locations, attention_weights, output, stream);
    }
}

size_t msda_backward_workspace_bytes(const msda_problem_t* problem) {
    if (check_problem(problem) != MSDA_SUCCESS) return 0;
    if (problem->dtype == MSDA_F32) return 0;
    return static_cast<size_t>(value_elems(problem)) * sizeof(float);
}

}  // extern "C"

namespace {

// The gradient kernel: accumulate into the float32 buffer gacc.
msda_status_t backward_kernel(const msda_problem_t* problem, const void* value,
                              const void* sampling_locations, const void* attention_weights,
                              const void* grad_output, float* gacc, void* grad_sampling_locations,
                              void* grad_attention_weights, hipStream_t stream) {
    if (out_elems(problem) == 0) return MSDA_SUCCESS;
    const msda::Problem pb = pack(problem);
    const LaneSplit s = lane_split(problem->embed_dims, problem->dtype);
    switch (problem->dtype) {
        case MSDA_F32:
            return by_split<kF32, Bwd>(s, pb, value, sampling_locations, attention_weights, grad_output,
                                       gacc, grad_sampling_locations, grad_attention_weights, stream);
        case MSDA_F16:
            return by_split<kF16, Bwd>(s, pb, value, sampling_locations, attention_weights, grad_output,
                                       gacc, grad_sampling_locations, grad_attention_weights, stream);
        default:
            return by_split<kBF16, Bwd>(s, pb, value, sampling_locations, attention_weights, grad_output,
                                        gacc, grad_sampling_locations, grad_attention_weights, stream);
    }
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

}  // namespace

extern "C" {

msda_status_t msda_backward(const msda_problem_t* problem, const void* value,
                            const void* sampling_locations, const void* attention_weights,
                            const void* grad_output, void* grad_value,
                            void* grad_sampling_locations, void* grad_attention_weights,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    MSDA_TRY(check_problem(problem));
    MSDA_TRY(check_backward_ptrs(problem, value, sampling_locations, attention_weights, grad_output,
                                 grad_value, grad_sampling_locations, grad_attention_weights));
    const int64_t nv = value_elems(problem);
    const size_t need = msda_backward_workspace_bytes(problem);
    if (need > 0) {
        if (workspace_bytes < need) return MSDA_ERROR_INVALID_VALUE;
        MSDA_TRY(check_ptr(workspace, nv));
    }
    if (nv == 0) return MSDA_SUCCESS;

    // grad_value rows that no sample touches must come back as zero.
    float* gacc = problem->dtype == MSDA_F32 ? static_cast<float*>(grad_value)
                                             : static_cast<float*>(workspace);
    const int64_t n16 = nv * 4 / 16;   // nv is a multiple of 8
    MSDA_TRY(launch(kfn(&msda::msda_zero_kernel), fill_blocks(n16), 0, stream,
                    reinterpret_cast<uint4*>(gacc), n16));

    MSDA_TRY(backward_kernel(problem, value, sampling_locations, attention_weights, grad_output, gacc,
                             grad_sampling_locations, grad_attention_weights, stream));

    if (problem->dtype != MSDA_F32) {
        const int64_t n8 = nv / 8;
        const void* k = problem->dtype == MSDA_F16 ? kfn(&msda::msda_narrow_kernel<kF16>)
                                                   : kfn(&msda::msda_narrow_kernel<kBF16>);
        MSDA_TRY(launch(k, fill_blocks(n8), 0, stream, reinterpret_cast<const float4*>(gacc),
                        static_cast<uint4*>(grad_value), n8));
    }
    return MSDA_SUCCESS;
}

msda_status_t msda_backward_accumulate(const msda_problem_t* problem, const void* value,
                                       const void* sampling_locations, const void* attention_weights,
                                       const void* grad_output, float* grad_value_acc,
                                       void* grad_sampling_locations, void* grad_attention_weights,
                                       hipStream_t stream) {
    MSDA_TRY(check_problem(problem));
    MSDA_TRY(check_backward_ptrs(problem, value, sampling_locations, attention_weights, grad_output,
                                 grad_value_acc, grad_sampling_locations, grad_attention_weights));
    return backward_kernel(problem, value, sampling_locations, attention_weights, grad_output,
                           grad_value_acc, grad_sampling_locations, grad_attention_weights, stream);
}

}  // extern "C"
