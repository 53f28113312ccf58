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
#include <type_traits>

#include "msda.h"
#include "msda_launch.hpp"

namespace {

using msda::kBF16;
using msda::kBlock;
using msda::kF16;
using msda::kF32;
using msda_host::count_chunks;
using msda_host::fused_count_scan;
using msda_host::kfn;
using msda_host::LaneSplit;
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

constexpr int64_t kIndexLimit = int64_t(1) << 31;

// Bytes of a value-side element (value, output and their gradients): 2
// for fp16, bf16 and the mixed codes, whose per-sample tensors are float32.
int elem_bytes(msda_dtype_t dt) { return dt == MSDA_F32 ? 4 : 2; }

msda_dtype_t value_dtype(msda_dtype_t dt) {
    return dt == MSDA_F16_F32 ? MSDA_F16 : dt == MSDA_BF16_F32 ? MSDA_BF16 : dt;
}

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
    if (p->dtype != MSDA_F32 && p->dtype != MSDA_F16 && p->dtype != MSDA_BF16 && p->dtype != MSDA_F16_F32 &&
        p->dtype != MSDA_BF16_F32)
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
    // Per batch, value and output bytes are addressed with 32-bit offsets.
    if (int64_t(p->num_keys) * pitch * elem_bytes(p->dtype) >= kIndexLimit) return MSDA_ERROR_NOT_SUPPORTED;
    if (int64_t(p->num_queries) * pitch * elem_bytes(p->dtype) >= kIndexLimit) return MSDA_ERROR_NOT_SUPPORTED;
    if (int64_t(p->num_queries) * p->num_heads * p->num_levels * p->num_points * 2 >= kIndexLimit)
        return MSDA_ERROR_NOT_SUPPORTED;
    return MSDA_SUCCESS;
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

int floor_log2(int64_t v) {
    int s = 0;
    while ((int64_t(2) << s) <= v) ++s;
    return s;
}

// Problem descriptor for the kernels, including the key segments of the
// binned backward: level l gets segments of 2^shift keys, sized so that a
// segment receives about 3/4 of a unit's records when the samples spread
// evenly over the level (two records per sample and level, Q*P samples per
// level and plane), but never fewer than 32 keys: a denser level spreads a
// segment over several units (merged with atomics) rather than letting
// many workers of one unit fold into the same few rows.  A tile of
// 2^shift keys * D floats stays within 32 KB (16 KB for sparse problems).
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
    pb.nplanes = p->batch * p->num_heads;
    // Sparse problems have many short units; they take smaller units and
    // tiles (16 KB instead of 32 KB), so that more units run per CU.  A
    // problem is sparse when its largest level gets fewer than one record per
    // key (two per sample, Q * P samples per level and plane): that level's
    // segments hold most of the units.
    int64_t largest = 0;
    for (int l = 0; l < p->num_levels; ++l)
        largest = std::max<int64_t>(largest, p->spatial_shapes[2 * l] * p->spatial_shapes[2 * l + 1]);
    const bool sparse = 2.0 * double(p->num_queries) * p->num_points < double(largest);
    pb.unit_records = sparse ? msda::kSparseUnitRecords : msda::kUnitRecords;
    const int max_shift = floor_log2(std::min<int64_t>(msda::kMaxSegKeys, (sparse ? 4096 : 8192) / p->embed_dims));
    int64_t nseg = 0;
    for (int l = 0; l < p->num_levels; ++l) {
        const int64_t H = p->spatial_shapes[2 * l], W = p->spatial_shapes[2 * l + 1];
        pb.lv.H[l] = static_cast<int32_t>(H);
        pb.lv.W[l] = static_cast<int32_t>(W);
        pb.lv.start[l] = static_cast<int32_t>(p->level_start_index[l]);
        const double per_key = 2.0 * double(p->num_queries) * p->num_points / double(H * W);
        const double keys = per_key > 0 ? (3 * pb.unit_records / 4) / per_key : double(msda::kMaxSegKeys);
        int shift = keys >= 1.0 ? floor_log2(static_cast<int64_t>(keys)) : 0;
        if (shift < 5) shift = 5;
        if (shift > max_shift) shift = max_shift;
        pb.seg_shift[l] = shift;
        pb.seg_base[l] = static_cast<int32_t>(std::min<int64_t>(nseg, kIndexLimit - 1));
        nseg += (H * W + (int64_t(1) << shift) - 1) >> shift;
    }
    pb.seg_base[p->num_levels] = static_cast<int32_t>(std::min<int64_t>(nseg, kIndexLimit - 1));
    pb.nseg = static_cast<int32_t>(std::min<int64_t>(nseg, kIndexLimit - 1));
    return pb;
}

// The binned backward needs: query indices within the record's 24-bit
// field, level extents within the 16-bit cell fields, at most kMaxSegments
// segments per plane, record positions and unit counts within int32.
int64_t max_records(const msda_problem_t* p) { return 4 * sample_elems(p); }

// Per plane: at most 4 records per sample, so a fixed region of
// plane_records; at most one unit per segment plus one per unit_records.
int64_t plane_records(const msda_problem_t* p) {
    return 4 * int64_t(p->num_queries) * p->num_levels * p->num_points;
}
int64_t plane_units(const msda_problem_t* p, const msda::Problem& pb) {
    return pb.nseg + (plane_records(p) + pb.unit_records - 1) / pb.unit_records;
}

bool binned_ok(const msda_problem_t* p, const msda::Problem& pb) {
    for (int l = 0; l < p->num_levels; ++l)
        if (p->spatial_shapes[2 * l] > msda::kMaxBinnedExtent || p->spatial_shapes[2 * l + 1] > msda::kMaxBinnedExtent)
            return false;
    return p->num_queries < (1 << msda::kQueryBits) && pb.nseg <= msda::kMaxSegments &&
           max_records(p) < kIndexLimit / 2 && int64_t(pb.nplanes) * plane_units(p, pb) < kIndexLimit / 2;
}

// ---- workspace layout --------------------------------------------------------

struct Layout {
    bool binned;
    size_t counts, cursor, nunits, multi, units, recs, acc, total;
    int64_t max_units;
};

size_t round_up(size_t v) { return (v + 255) & ~size_t(255); }

Layout layout(const msda_problem_t* p, const msda::Problem& pb) {
    Layout w;
    memset(&w, 0, sizeof(w));
    w.binned = binned_ok(p, pb);
    size_t off = 0;
    if (w.binned) {
        const int64_t nbins = int64_t(pb.nplanes) * pb.nseg;
        w.max_units = int64_t(pb.nplanes) * plane_units(p, pb);
        // one histogram row per counting workgroup
        w.counts = off;
        if (!fused_count_scan(pb)) off += round_up(nbins * count_chunks(pb) * 4);
        w.cursor = off;
        off += round_up(nbins * 4);
        // [p] units of plane p, [nplanes + p] its multi-unit segments (both
        // from the scan), [2 nplanes + p] units before plane p and
        // [3 nplanes] all units (from the gradient kernel)
        w.nunits = off;
        off += round_up((size_t(pb.nplanes) * 3 + 1) * 4);
        w.multi = off;
        off += round_up(nbins * 4);
        w.units = off;
        off += round_up(w.max_units * 16);
        w.recs = off;
        off += round_up(max_records(p) * 12);
    }
    w.acc = off;
    if (p->dtype != MSDA_F32) off += round_up(value_elems(p) * 4);
    w.total = off;
    return w;
}

// A device pointer must be non-NULL when its tensor has elements, and
// 16-byte aligned when non-NULL.
msda_status_t check_ptr(const void* ptr, int64_t elems) {
    if (elems > 0 && ptr == nullptr) return MSDA_ERROR_INVALID_VALUE;
    if (ptr != nullptr && !aligned16(ptr)) return MSDA_ERROR_MISALIGNED;
    return MSDA_SUCCESS;
}

int64_t fill_blocks(int64_t n) {
    const int64_t want = (n + kBlock - 1) / kBlock;
    return want < 8192 ? (want > 0 ? want : 1) : 8192;
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

msda_status_t forward_call(const msda_problem_t* problem, int ref_dims, const void* value, const void* ref,
                           const uint8_t* kmask, const void* sampling_locations, const void* attention_weights,
                           void* output, hipStream_t stream) {
    MSDA_TRY(check_problem(problem));
    MSDA_TRY(check_ref(problem, ref_dims, ref));
    MSDA_TRY(check_ptr(value, value_elems(problem)));
    MSDA_TRY(check_ptr(sampling_locations, sample_elems(problem)));
    MSDA_TRY(check_ptr(attention_weights, sample_elems(problem)));
    MSDA_TRY(check_ptr(output, out_elems(problem)));
    if (out_elems(problem) == 0) return MSDA_SUCCESS;
    const msda::Problem pb = pack(problem);
    const LaneSplit s = lane_split(problem->embed_dims, problem->dtype);
    return by_code(problem->dtype, [&](auto c) {
        return Launch<decltype(c)::value>::forward(s, pb, ref_dims, value, ref, kmask, sampling_locations,
                                                   attention_weights, output, stream);
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
                         int4* units, int accumulate, int plane_recs, int plane_us, hipEvent_t* ev, hipStream_t st) {
    return by_code(dt, [&](auto c) {
        return Launch<decltype(c)::value>::count_scan(pb, ref_dims, ref, loc, counts, cursor, nunits, multi, units,
                                                      accumulate, plane_recs, plane_us, ev, st);
    });
}

// The backward.  accumulate = 1: grad_value is added into the float32
// buffer gacc (gfinal unused).  accumulate = 0: grad_value is overwritten
// into gfinal, the caller's tensor of the problem's dtype; gacc is gfinal for
// float32 and the workspace's float32 buffer for 16-bit dtypes, which then
// holds only rows the kernels add into (and is rounded into gfinal at the
// end).
// ref_dims != 0: the fused prologue (loc and w are the offsets and logits,
// gloc and gw receive their gradients).
msda_status_t backward_into(const msda_problem_t* problem, int ref_dims, const void* value, const void* ref,
                            const uint8_t* kmask, const void* loc, const void* w, const void* gout, float* gacc,
                            void* gfinal, void* gloc, void* gw, char* ws, int accumulate, hipEvent_t* ev,
                            hipStream_t st) {
    const bool narrow16 = !accumulate && problem->dtype != MSDA_F32;
    if (sample_elems(problem) == 0) {
        // no samples (Q = 0): grad_value is zero and nothing else is written
        MSDA_TRY(mark(ev, kStageZero, st));
        if (!accumulate)
            MSDA_TRY(zero_bytes(gfinal, size_t(value_elems(problem)) * (problem->dtype == MSDA_F32 ? 4 : 2), st));
        for (int stage = kStageCount; stage <= kStageNarrow; ++stage) MSDA_TRY(mark(ev, stage, st));
        return MSDA_SUCCESS;
    }
    const msda::Problem pb = pack(problem);
    const Layout lay = layout(problem, pb);
    const LaneSplit s = lane_split(problem->embed_dims, problem->dtype);
    if (!lay.binned) {
        // Float atomics straight into gacc.
        MSDA_TRY(mark(ev, kStageZero, st));
        if (!accumulate) MSDA_TRY(zero_bytes(gacc, size_t(value_elems(problem)) * 4, st));
        MSDA_TRY(mark(ev, kStageCount, st));
        MSDA_TRY(mark(ev, kStageScan, st));
        MSDA_TRY(mark(ev, kStageGrad, st));
        MSDA_TRY(gradient(problem->dtype, s, pb, false, ref_dims, value, ref, kmask, loc, w, gout, gacc,
                                      static_cast<uint3*>(nullptr), static_cast<int32_t*>(nullptr),
                                      static_cast<int32_t*>(nullptr), static_cast<const int32_t*>(nullptr),
                                      gloc, gw, st));
        MSDA_TRY(mark(ev, kStageAccum, st));
        MSDA_TRY(mark(ev, kStageNarrow, st));
        if (narrow16) {
            const int64_t n8 = value_elems(problem) / 8;
            const void* k = value_dtype(problem->dtype) == MSDA_F16 ? kfn(&msda::msda_narrow_kernel<kF16>)
                                                       : kfn(&msda::msda_narrow_kernel<kBF16>);
            MSDA_TRY(launch(k, fill_blocks(n8), kBlock, 0, st, reinterpret_cast<const float4*>(gacc),
                            static_cast<uint4*>(gfinal), n8));
        }
        return MSDA_SUCCESS;
    }
    int32_t* counts = reinterpret_cast<int32_t*>(ws + lay.counts);
    int32_t* cursor = reinterpret_cast<int32_t*>(ws + lay.cursor);
    int32_t* nunits = reinterpret_cast<int32_t*>(ws + lay.nunits);
    int32_t* multi = reinterpret_cast<int32_t*>(ws + lay.multi);
    int4* units = reinterpret_cast<int4*>(ws + lay.units);
    uint3* recs = reinterpret_cast<uint3*>(ws + lay.recs);

    MSDA_TRY(mark(ev, kStageZero, st));             // no zero fill on this path
    const int prec = static_cast<int>(plane_records(problem)), pun = static_cast<int>(plane_units(problem, pb));
    MSDA_TRY(count_scan(problem->dtype, pb, ref_dims, ref, loc, counts, cursor, nunits, multi, units, accumulate,
                        prec, pun, ev, st));
    MSDA_TRY(mark(ev, kStageGrad, st));
    MSDA_TRY(gradient(problem->dtype, s, pb, true, ref_dims, value, ref, kmask, loc, w, gout, gacc, recs,
                                  cursor,
                                  nunits, static_cast<const int32_t*>(multi), gloc, gw,
                                  st));
    MSDA_TRY(mark(ev, kStageAccum, st));
    MSDA_TRY(accumulate_rows(problem->dtype, s, pb, lay.max_units, static_cast<int>(plane_units(problem, pb)),
                                   gout, static_cast<const uint3*>(recs), static_cast<const int32_t*>(nunits),
                                   static_cast<const int4*>(units), kmask, gacc, narrow16 ? gfinal : nullptr, st));
    MSDA_TRY(mark(ev, kStageNarrow, st));
    if (narrow16) {
        const void* k = value_dtype(problem->dtype) == MSDA_F16 ? kfn(&msda::msda_narrow_segments_kernel<kF16>)
                                                   : kfn(&msda::msda_narrow_segments_kernel<kBF16>);
        MSDA_TRY(launch(k, int64_t(pb.nplanes) * msda::kNarrowPerPlane, kBlock, 0, st,
                        static_cast<const float*>(gacc), gfinal, static_cast<const int32_t*>(nunits),
                        static_cast<const int32_t*>(multi), pb));
    }
    return MSDA_SUCCESS;
}

msda_status_t backward_call(const msda_problem_t* problem, int ref_dims, const void* value, const void* ref,
                            const uint8_t* kmask, const void* sampling_locations, const void* attention_weights,
                            const void* grad_output, void* grad_value, void* grad_sampling_locations,
                            void* grad_attention_weights, void* workspace, size_t workspace_bytes, hipEvent_t* ev,
                            hipStream_t stream) {
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
                           gacc, grad_value, grad_sampling_locations, grad_attention_weights, ws, 0, ev, stream));
    return mark(ev, kStageEnd, stream);
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
    return forward_call(problem, 0, value, nullptr, nullptr, sampling_locations, attention_weights, output, stream);
}

msda_status_t msda_forward_fused(const msda_problem_t* problem, int32_t ref_dims, const void* value,
                                 const uint8_t* key_padding_mask, const void* reference_points,
                                 const void* sampling_offsets, const void* attention_logits, void* output,
                                 hipStream_t stream) {
    if (ref_dims != 2 && ref_dims != 4) return MSDA_ERROR_INVALID_VALUE;
    return forward_call(problem, ref_dims, value, reference_points, key_padding_mask, sampling_offsets,
                        attention_logits, output, stream);
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
                         static_cast<char*>(workspace), 1, nullptr, stream);
}

}  // extern "C"
