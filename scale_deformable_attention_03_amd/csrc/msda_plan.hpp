// Host planning of the MSDeformAttn calls: descriptor validation, the
// kernels' problem descriptor (level table, key segments of the binned
// backward), lane split, workspace layout and the backward's launch plan.
// Plain C++ (no HIP calls, no device code), so that the tests also build it
// with a host compiler under AddressSanitizer and UndefinedBehaviorSanitizer
// and fuzz it across the envelope's edges on the CPU.  Internal to the
// library; msda_api.hip and the launch code use these functions, so the
// plan tested on the CPU is the plan the library launches.
#pragma once

#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "msda.h"
#include "msda_types.hpp"

namespace msda_plan {

constexpr int64_t kIndexLimit = int64_t(1) << 31;

// Bytes of a value-side element (value, output and their gradients): 2
// for fp16, bf16 and the mixed codes, whose per-sample tensors are float32.
inline int elem_bytes(msda_dtype_t dt) { return dt == MSDA_F32 ? 4 : 2; }

inline msda_dtype_t value_dtype(msda_dtype_t dt) {
    return dt == MSDA_F16_F32 ? MSDA_F16 : dt == MSDA_BF16_F32 ? MSDA_BF16 : dt;
}

// Lane split of one group: VECB bytes per lane, LPR lanes (a power of two,
// at least 4) of which `active` own channels.
struct LaneSplit {
    int vecb, lpr, active;
};

inline LaneSplit lane_split(int embed_dims, msda_dtype_t dt) {
    const int row = embed_dims * elem_bytes(dt);   // a multiple of 16 bytes
    LaneSplit s;
    s.vecb = row >= 64 ? 16 : (row % 8 == 0 && row >= 32 ? 8 : 4);
    s.active = row / s.vecb;
    s.lpr = 4;
    while (s.lpr < s.active) s.lpr *= 2;
    return s;
}

inline msda_status_t check_problem(const msda_problem_t* p) {
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

inline int64_t value_elems(const msda_problem_t* p) {
    return int64_t(p->batch) * p->num_keys * p->num_heads * p->embed_dims;
}
inline int64_t sample_elems(const msda_problem_t* p) {
    return int64_t(p->batch) * p->num_queries * p->num_heads * p->num_levels * p->num_points;
}
inline int64_t out_elems(const msda_problem_t* p) {
    return int64_t(p->batch) * p->num_queries * p->num_heads * p->embed_dims;
}

inline int floor_log2(int64_t v) {
    int s = 0;
    while ((int64_t(2) << s) <= v) ++s;
    return s;
}

// Problem descriptor for the kernels (of a valid descriptor), including the
// key segments of the binned backward: level l gets segments of 2^shift
// keys, sized so that a segment receives about 3/4 of a unit's records when
// the samples spread evenly over the level (two records per sample and
// level, Q*P samples per level and plane), but never fewer than 32 keys: a
// denser level spreads a segment over several units (merged with atomics)
// rather than letting many workers of one unit fold into the same few rows.
// A tile of 2^shift keys * D floats stays within 32 KB (16 KB for sparse
// problems).
inline msda::Problem pack(const msda_problem_t* p) {
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
        int shift = keys >= 1.0 ? floor_log2(static_cast<int64_t>(std::min(keys, 1e18))) : 0;
        if (shift < 5) shift = 5;
        if (shift > max_shift) shift = max_shift;
        pb.seg_shift[l] = shift;
        pb.seg_base[l] = static_cast<int32_t>(std::min<int64_t>(nseg, kIndexLimit - 1));
        nseg += (H * W + (int64_t(1) << shift) - 1) >> shift;
    }
    pb.seg_base[p->num_levels] = static_cast<int32_t>(std::min<int64_t>(nseg, kIndexLimit - 1));
    pb.nseg = static_cast<int32_t>(std::min<int64_t>(nseg, kIndexLimit - 1));
    // Record merging (msda_device.hpp) on planes counted apart from the scan:
    // on the small planes that one workgroup counts and scans, its extra
    // work costs more than the records it saves (decoder: 6% fewer records,
    // step 46.4 -> 49.2 us with merging)
    pb.merge_records = int64_t(p->num_queries) * p->num_levels * p->num_points > msda::kCountScanSamples ? 1 : 0;
    return pb;
}

// The binned backward needs: query indices within the record's 24-bit
// field, level extents within the 16-bit cell fields, at most kMaxSegments
// segments per plane, record positions and unit counts within int32.
inline int64_t max_records(const msda_problem_t* p) { return 4 * sample_elems(p); }

// Per plane: at most 4 records per sample, so a fixed region of
// plane_records; at most one unit per segment plus one per unit_records.
inline int64_t plane_records(const msda_problem_t* p) {
    return 4 * int64_t(p->num_queries) * p->num_levels * p->num_points;
}
inline int64_t plane_units(const msda_problem_t* p, const msda::Problem& pb) {
    return pb.nseg + (plane_records(p) + pb.unit_records - 1) / pb.unit_records;
}

inline bool binned_ok(const msda_problem_t* p, const msda::Problem& pb) {
    for (int l = 0; l < p->num_levels; ++l)
        if (p->spatial_shapes[2 * l] > msda::kMaxBinnedExtent || p->spatial_shapes[2 * l + 1] > msda::kMaxBinnedExtent)
            return false;
    return p->num_queries < (1 << msda::kQueryBits) && pb.nseg <= msda::kMaxSegments &&
           max_records(p) < kIndexLimit / 2 && int64_t(pb.nplanes) * plane_units(p, pb) < kIndexLimit / 2;
}

// Counting: samples per counting workgroup (one histogram row each) and the
// number of rows per plane; planes of at most kCountScanSamples samples are
// counted and scanned by one workgroup instead (no rows).  At most
// kMaxCountChunks rows per plane; workgroups of kCountChunk samples when the
// plane has at most one segment per scan lane, of twice that otherwise
// (measured: 4096-sample chunks shorten the encoder's count by 3.7 us for
// 0.5 us more scan; with 842 segments per plane the fp16 stress workload's
// scan grew by 6 us for 4 us less count).
inline int64_t count_chunk(const msda::Problem& pb) {
    const int64_t nsamp = int64_t(pb.Q) * pb.L * pb.P;
    const int64_t chunk = pb.nseg <= msda::kBlock ? msda::kCountChunk : 2 * msda::kCountChunk;
    // a multiple of 4 samples: the count loads 2 or 4 consecutive samples at
    // once, and record merging needs a level's four points in one lane pair
    return (std::max<int64_t>(chunk, (nsamp + msda::kMaxCountChunks - 1) / msda::kMaxCountChunks) + 3) & ~int64_t(3);
}
inline int64_t count_chunks(const msda::Problem& pb) {
    const int64_t nsamp = int64_t(pb.Q) * pb.L * pb.P;
    return (nsamp + count_chunk(pb) - 1) / count_chunk(pb);
}
inline bool fused_count_scan(const msda::Problem& pb) {
    return int64_t(pb.Q) * pb.L * pb.P <= msda::kCountScanSamples;
}

inline int64_t plane_blocks(const msda::Problem& pb, int gpb) {
    return int64_t(pb.nplanes) * ((pb.Q + gpb - 1) / gpb);
}

// Queries per workgroup: the full 256 lanes unless the per-sample LDS
// records would exceed `max_samples` samples per workgroup.  With `shrink`,
// small problems (fewer than two workgroups per compute unit) take smaller
// workgroups, down to one wave, so that more compute units share the
// latency-bound work.
inline int tile_queries(const msda::Problem& pb, int lpr, int max_samples, bool shrink) {
    constexpr int64_t kFill = 2 * 256;
    int gpb = msda::kBlock / lpr;
    const int cap = max_samples / (pb.L * pb.P);
    if (gpb > cap) gpb = cap < 1 ? 1 : cap;
    while (shrink && plane_blocks(pb, gpb) < kFill && gpb * lpr > 64 && gpb % 2 == 0) gpb /= 2;
    return gpb;
}

// Queries per gradient workgroup (full workgroups: measured, the
// per-workgroup cursor reservation makes smaller ones slower on small
// problems).
inline int grad_tile(const msda::Problem& pb, int lpr) { return tile_queries(pb, lpr, msda::kMaxWgSamples, false); }

// ---- workspace layout --------------------------------------------------------

struct Layout {
    bool binned;
    size_t counts, cursor, nunits, multi, units, recs, acc, total;
    int64_t max_units;
};

inline size_t round_up(size_t v) { return (v + 255) & ~size_t(255); }

inline Layout layout(const msda_problem_t* p, const msda::Problem& pb) {
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

// ---- the backward's launches --------------------------------------------------

// Grid sizes of the backward's launches in order (0 = not launched), for a
// valid descriptor.  accumulate: add into a float32 buffer instead of
// overwriting grad_value.
struct BackwardPlan {
    bool binned;
    int64_t zero_blocks;        // zero fill of grad_value (empty problems) or of the float32 rows (atomic path)
    int64_t count_blocks;       // counting workgroups (0 when one kernel counts and scans)
    int64_t scan_blocks;        // scan, or count+scan, one workgroup per plane
    int64_t grad_blocks;        // the gradient kernel
    int64_t accum_blocks;       // the accumulation (bound; extra workgroups exit)
    int64_t narrow_blocks;      // rounding of float32 rows to 16 bits
};

inline int64_t fill_blocks(int64_t n) {
    const int64_t want = (n + msda::kBlock - 1) / msda::kBlock;
    return want < 8192 ? (want > 0 ? want : 1) : 8192;
}

inline BackwardPlan plan_backward(const msda_problem_t* p, bool accumulate) {
    BackwardPlan b;
    memset(&b, 0, sizeof(b));
    const bool narrow16 = !accumulate && p->dtype != MSDA_F32;
    if (value_elems(p) == 0) return b;
    if (sample_elems(p) == 0) {
        // no samples (Q = 0): grad_value is zero and nothing else is written
        if (!accumulate) b.zero_blocks = fill_blocks(value_elems(p) * (p->dtype == MSDA_F32 ? 4 : 2) / 16);
        return b;
    }
    const msda::Problem pb = pack(p);
    const Layout lay = layout(p, pb);
    const LaneSplit s = lane_split(p->embed_dims, p->dtype);
    b.binned = lay.binned;
    b.grad_blocks = plane_blocks(pb, grad_tile(pb, s.lpr));
    if (!lay.binned) {
        if (!accumulate) b.zero_blocks = fill_blocks(value_elems(p) * 4 / 16);
        if (narrow16) b.narrow_blocks = fill_blocks(value_elems(p) / 8);
        return b;
    }
    if (fused_count_scan(pb)) {
        b.scan_blocks = pb.nplanes;
    } else {
        b.count_blocks = int64_t(pb.nplanes) * count_chunks(pb);
        b.scan_blocks = pb.nplanes;
    }
    // the accumulation reads the unit prefix that the gradient kernel's
    // workgroup 0 writes: never planned without a gradient launch
    b.accum_blocks = b.grad_blocks > 0 ? lay.max_units : 0;
    if (narrow16) b.narrow_blocks = int64_t(pb.nplanes) * msda::kNarrowPerPlane;
    return b;
}

}  // namespace msda_plan
