// Definitions of the per-dtype launch functions: launch shapes, kernel
// selection and the launches.  Included only by the translation units that
// instantiate the kernels (msda_kernels_<dtype>.hip).  Internal.
#pragma once

#include "msda_launch.hpp"

namespace msda_host {

// ---- kernel selection ----------------------------------------------------------

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

inline bool is_l4p4(const msda::Problem& pb) { return pb.L == 4 && pb.P == 4; }
// four levels of 16 points (L * P = 64, the envelope's maximum): a
// fixed-size gradient kernel for the plain form, so that samples batch their
// loads as for L4P4 (measured: 127 -> 92 us on the fp16 stress workload; the
// forward gained nothing from it and stays generic)
inline bool is_l4p16(const msda::Problem& pb) { return pb.L == 4 && pb.P == 16; }

using msda_plan::grad_tile;
using msda_plan::plane_blocks;
using msda_plan::tile_queries;

// Reference-point form of a call: 0 (locations and weights given), 2 or 4
// (reference points, offsets and logits given; the fused prologue).
template <int DT, int VECB, int LPR, int REF, bool CNT = false>
const void* fwd_kernel(const msda::Problem& pb) {
    return is_l4p4(pb) ? kfn(&msda::msda_forward_kernel<DT, VECB, LPR, 4, 4, REF, CNT>)
                       : kfn(&msda::msda_forward_kernel<DT, VECB, LPR, 0, 0, REF, CNT>);
}

template <int DT, int VECB, int LPR, bool BINNED, int REF>
const void* grad_kernel(const msda::Problem& pb) {
    if constexpr (REF == 0)
        if (is_l4p16(pb)) return kfn(&msda::msda_backward_kernel<DT, VECB, LPR, 4, 16, BINNED, REF>);
    return is_l4p4(pb) ? kfn(&msda::msda_backward_kernel<DT, VECB, LPR, 4, 4, BINNED, REF>)
                       : kfn(&msda::msda_backward_kernel<DT, VECB, LPR, 0, 0, BINNED, REF>);
}

// LDS of the fused prologue: logits and their exponentials.
inline size_t fused_lds(int ref_dims, int gpb, int LP) { return ref_dims ? sizeof(float) * 2 * size_t(gpb) * LP : 0; }

template <int DT, int VECB, int LPR>
struct Fwd {
    // counts != null (plain form only): the forward also counts the
    // backward's records into the zeroed histogram rows `counts`
    static msda_status_t run(const msda::Problem& pb, int ref_dims, const void* v, const void* ref,
                             const uint8_t* kmask, const void* loc, const void* w, void* out, int32_t* counts,
                             int nchunks, hipStream_t st) {
        if (counts != nullptr && ref_dims != 0) return MSDA_ERROR_INVALID_VALUE;
        const int gpb = tile_queries(pb, LPR, 1024, true);
        const int LP = pb.L * pb.P;
        size_t lds = sizeof(uint32_t) * gpb * (8 * LP + 4) + fused_lds(ref_dims, gpb, LP);
        if (counts != nullptr) lds += sizeof(int32_t) * size_t(pb.nseg);
        const void* k = counts != nullptr ? fwd_kernel<DT, VECB, LPR, 0, true>(pb)
                        : ref_dims == 0   ? fwd_kernel<DT, VECB, LPR, 0>(pb)
                        : ref_dims == 2   ? fwd_kernel<DT, VECB, LPR, 2>(pb)
                                          : fwd_kernel<DT, VECB, LPR, 4>(pb);
        return launch(k, plane_blocks(pb, gpb), gpb * LPR, lds, st, v, loc, w, ref, kmask, out, pb, gpb, counts,
                      nchunks);
    }
};

template <int DT, int VECB, int LPR>
struct Grad {
    static msda_status_t run(const msda::Problem& pb, bool binned, int ref_dims, const void* v, const void* ref,
                             const uint8_t* kmask, const void* loc, const void* w, const void* gout, float* gacc,
                             uint3* recs,
                             int32_t* cursor, int32_t* nunits, const int32_t* multi, void* gloc, void* gw,
                             hipStream_t st) {
        const int gpb = grad_tile(pb, LPR);
        const int LP = pb.L * pb.P;
        const int64_t blocks = plane_blocks(pb, gpb);
        size_t lds = sizeof(uint32_t) * gpb * (8 * LP + 4) + fused_lds(ref_dims, gpb, LP);
        if (binned) lds += sizeof(int32_t) * 2 * size_t(pb.nseg);
        else  // the pre-reduction: grad_output rows, bucket starts and ends, entry ids
            lds += sizeof(float) * size_t(gpb) * pb.D + sizeof(int32_t) * 2 * msda::kPreBuckets +
                   sizeof(uint16_t) * 4 * size_t(gpb) * LP;
        const void* k;
        if (binned)
            k = ref_dims == 0   ? grad_kernel<DT, VECB, LPR, true, 0>(pb)
                : ref_dims == 2 ? grad_kernel<DT, VECB, LPR, true, 2>(pb)
                                : grad_kernel<DT, VECB, LPR, true, 4>(pb);
        else
            k = ref_dims == 0   ? grad_kernel<DT, VECB, LPR, false, 0>(pb)
                : ref_dims == 2 ? grad_kernel<DT, VECB, LPR, false, 2>(pb)
                                : grad_kernel<DT, VECB, LPR, false, 4>(pb);
        return launch(k, blocks, gpb * LPR, lds, st, v, loc, w, ref, kmask, gout, gacc, recs, cursor, nunits,
                      multi, gloc, gw, pb, gpb);
    }
};

template <int DT, int VECB, int LPR>
struct Accum {
    template <int UNIT>
    static msda_status_t go(const msda::Problem& pb, int64_t max_units, int plane_units, const void* gout,
                            const uint3* recs, const int32_t* nunits, const int4* units, const uint8_t* kmask,
                            float* gacc, void* gfinal, hipStream_t st) {
        int max_shift = 0;
        for (int l = 0; l < pb.L; ++l) max_shift = pb.seg_shift[l] > max_shift ? pb.seg_shift[l] : max_shift;
        const size_t lds = sizeof(float) * (size_t(1) << max_shift) * pb.D +
                           sizeof(float2) * msda::sorted_pair_slots(UNIT) +
                           sizeof(uint32_t) * msda::sorted_key_slots(UNIT) + 2 * sizeof(int32_t) * msda::kMaxSegKeys;
        return launch(kfn(&msda::msda_accumulate_kernel<DT, VECB, LPR, UNIT>), max_units, msda::acc_block(LPR, UNIT),
                      lds, st, gout, recs, nunits, units, kmask, gacc, gfinal, pb, plane_units);
    }
    static msda_status_t run(const msda::Problem& pb, int64_t max_units, int plane_units, const void* gout,
                             const uint3* recs, const int32_t* nunits, const int4* units, const uint8_t* kmask,
                             float* gacc, void* gfinal, hipStream_t st) {
        return pb.unit_records == msda::kSparseUnitRecords
                   ? go<msda::kSparseUnitRecords>(pb, max_units, plane_units, gout, recs, nunits, units, kmask, gacc,
                                                  gfinal, st)
                   : go<msda::kUnitRecords>(pb, max_units, plane_units, gout, recs, nunits, units, kmask, gacc,
                                            gfinal, st);
    }
};

template <int DT, int REF>
const void* count_kernel(const msda::Problem& pb) {
    return is_l4p4(pb) ? kfn(&msda::msda_bin_count_kernel<DT, 4, 4, REF>)
                       : kfn(&msda::msda_bin_count_kernel<DT, 0, 0, REF>);
}

template <int DT, int REF>
const void* count_scan_kernel(const msda::Problem& pb) {
    return is_l4p4(pb) ? kfn(&msda::msda_bin_count_scan_kernel<DT, 4, 4, REF>)
                       : kfn(&msda::msda_bin_count_scan_kernel<DT, 0, 0, REF>);
}

// Count records per segment and scan the counts into ranges, cursors and
// units: one fused launch for small planes, else count (histogram rows) and
// scan.  Events: the count stage before, the scan stage between.
// counted: the histogram rows were filled by a counting forward (not for
// small planes, which count and scan in one launch), so only the scan runs.
template <int DT>
msda_status_t count_scan_launch(const msda::Problem& pb, int ref_dims, const void* ref, const void* loc,
                                int32_t* counts, int32_t* cursor, int32_t* nunits, int32_t* multi, int4* units,
                                int accumulate, int plane_recs, int plane_us, bool counted, hipEvent_t* ev,
                                hipStream_t st) {
    MSDA_TRY(mark(ev, kStageCount, st));
    if (fused_count_scan(pb)) {
        const void* k = ref_dims == 0   ? count_scan_kernel<DT, 0>(pb)
                        : ref_dims == 2 ? count_scan_kernel<DT, 2>(pb)
                                        : count_scan_kernel<DT, 4>(pb);
        MSDA_TRY(launch(k, pb.nplanes, msda::kCountScanBlock, 0, st, loc, ref, cursor, nunits, multi, units,
                        accumulate, pb, plane_recs, plane_us));
        return mark(ev, kStageScan, st);
    }
    const int64_t chunks = count_chunks(pb);
    if (!counted) {
        const void* k = ref_dims == 0   ? count_kernel<DT, 0>(pb)
                        : ref_dims == 2 ? count_kernel<DT, 2>(pb)
                                        : count_kernel<DT, 4>(pb);
        MSDA_TRY(launch(k, int64_t(pb.nplanes) * chunks, msda::kCountBlock, sizeof(int32_t) * pb.nseg, st, loc,
                        ref, counts, pb, static_cast<int>(count_chunk(pb))));
    }
    MSDA_TRY(mark(ev, kStageScan, st));
    return launch(kfn(&msda::msda_bin_scan_kernel), pb.nplanes, msda::kScanBlock, 0, st,
                  static_cast<const int32_t*>(counts), counted ? msda::kForwardCountRows : static_cast<int>(chunks),
                  cursor, nunits, multi, units,
                  accumulate, pb, plane_recs, plane_us);
}



template <int DT>
msda_status_t Launch<DT>::forward(const LaneSplit& s, const msda::Problem& pb, int ref_dims, const void* v,
                                  const void* ref, const uint8_t* kmask, const void* loc, const void* w, void* out,
                                  int32_t* counts, int nchunks, hipStream_t st) {
    return by_split<DT, Fwd>(s, pb, ref_dims, v, ref, kmask, loc, w, out, counts, nchunks, st);
}

template <int DT>
msda_status_t Launch<DT>::gradient(const LaneSplit& s, const msda::Problem& pb, bool binned, int ref_dims,
                                   const void* v, const void* ref, const uint8_t* kmask, const void* loc,
                                   const void* w, const void* gout, float* gacc, uint3* recs, int32_t* cursor,
                                   int32_t* nunits, const int32_t* multi, void* gloc, void* gw, hipStream_t st) {
    return by_split<DT, Grad>(s, pb, binned, ref_dims, v, ref, kmask, loc, w, gout, gacc, recs, cursor, nunits,
                              multi, gloc, gw, st);
}

template <int DT>
msda_status_t Launch<DT>::accumulate(const LaneSplit& s, const msda::Problem& pb, int64_t max_units,
                                     int plane_units, const void* gout, const uint3* recs, const int32_t* nunits,
                                     const int4* units, const uint8_t* kmask, float* gacc, void* gfinal,
                                     hipStream_t st) {
    if constexpr (msda::value_dt(DT) != kF32) {
        // Short 16-bit rows (32 to 64 bytes) fold with 8-byte lanes (4
        // elements each): twice the lanes of the gather kernels' 16-byte
        // split, so a unit's workgroup has as many waves as in float32 and
        // each lane the same fold work per record (measured: bf16 D = 32
        // accumulation 118 -> 99 us on the encoder shapes).  Longer rows keep
        // the 16-byte split: at D = 64, 16 lanes per worker made 1024-lane
        // workgroups and a slower accumulation (271 -> 367 us).
        const int row = pb.D * 2;
        if (row >= 32 && row <= 64 && row % 8 == 0) {
            msda::Problem pa = pb;
            pa.lpr_active = row / 8;
            return row / 8 <= 4 ? Accum<DT, 8, 4>::run(pa, max_units, plane_units, gout, recs, nunits, units, kmask,
                                                       gacc, gfinal, st)
                                : Accum<DT, 8, 8>::run(pa, max_units, plane_units, gout, recs, nunits, units, kmask,
                                                       gacc, gfinal, st);
        }
    }
    return by_split<DT, Accum>(s, pb, max_units, plane_units, gout, recs, nunits, units, kmask, gacc, gfinal, st);
}

template <int DT>
msda_status_t Launch<DT>::count_scan(const msda::Problem& pb, int ref_dims, const void* ref, const void* loc,
                                     int32_t* counts, int32_t* cursor, int32_t* nunits, int32_t* multi, int4* units,
                                     int accumulate, int plane_recs, int plane_us, bool counted, hipEvent_t* ev,
                                     hipStream_t st) {
    return count_scan_launch<DT>(pb, ref_dims, ref, loc, counts, cursor, nunits, multi, units, accumulate,
                                 plane_recs, plane_us, counted, ev, st);
}

}  // namespace msda_host
