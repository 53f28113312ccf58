// MSDeformAttn core backward for gfx950.
//
// What is differentiated: the forward of "Deformable DETR walkthrough"
// (zhangshiyu.com/post/59697), section 2.2.4 (bilinear grid_sample with zero
// padding, align_corners=False, weighted and summed over levels and points);
// the gradients are those MSDeformAttnFunction.backward returns on the
// "DQ-DETR ops directory" CSDN page, section 2(3): value, sampling
// locations, attention weights.
//
// grad_attention_weights and grad_sampling_locations are per-sample
// reductions over the embedding channels, computed by the gradient kernel,
// which gathers the four corner rows exactly as the forward does.  With
// d_ij = <g, v_ij> (g the sample's grad_output row, v_ij its corners) the
// three reductions follow from four dot products:
//   grad_w   = hy (hx d00 + lx d01) + ly (hx d10 + lx d11)
//   grad_x   = W w (hy (d01 - d00) + ly (d11 - d10))
//   grad_y   = H w ((hx d10 + lx d11) - (hx d00 + lx d01))
//
// grad_value is a transposed gather: row (b, key, m) sums w * (bilinear
// weight) * grad_output[b, q, m] over every sample corner that lands on it.
// Scattering those D-wide contributions with float atomics costs one L2
// atomic per element per sample corner: on MI355X the scatter kernel of
// msda_micro.hip adds the DETR encoder's 584 M such updates at 68-119 G/s
// (4.9-8.6 ms), against well under a millisecond for the whole binned
// backward.  So the backward bins instead:
//
//   1. count     each (batch, head) plane's keys are cut into segments; the
//                in-map corners of one image row of a sample's cell make a
//                record; count records per segment (an LDS histogram per
//                workgroup, written out as that workgroup's row of counts).
//                In a training step the forward kernel (CNT) counts them
//                instead, from the cells it computes anyway, adding into one
//                zeroed row per plane; the backward then starts at the scan.
//   2. scan      sum the rows, then an exclusive prefix over the counts gives
//                each segment a record range and a cursor (small planes count
//                and scan in one kernel); segments are split into units of at most
//                unit_records (kUnitRecords, or kSparseUnitRecords for sparse
//                problems) records.
//   3. gradient  the gather kernel (grad_w, grad_loc) also writes its records
//                at positions reserved per workgroup and segment: the query
//                and key (4 bytes) and the two corner weights (8 bytes).
//   4. accumulate  one workgroup per unit: counting-sort the unit's records by
//                key in LDS, let each worker (LPR lanes) walk a key-sorted slice
//                accumulating rows in registers, merge into an LDS tile, and
//                write every row of the segment once with plain stores (units
//                of a segment split in several use float atomics instead, into
//                rows the gradient kernel zeroed).
//
// Segment sizes per level are planned on the host from the expected records
// per key, so that most segments fit one unit.  Outside the envelope of the
// record format (binned_ok on the host) the gradient kernel scatters
// grad_value with float atomics instead, after merging its own corners that
// share a row (pre_reduce_scatter).
#pragma once

#include "msda_device.hpp"
#include "msda_forward.hpp"

namespace msda {

// Level of plane-local segment `seg`.
__device__ __forceinline__ int level_of_segment(const Problem& pb, int seg) {
    int l = 0;
    while (l + 1 < pb.L && seg >= pb.seg_base[l + 1]) ++l;
    return l;
}

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------

// Zero n16 16-byte words (a kernel, not a memset node, so that the backward
// stays correct inside a captured HIP graph).
[[maybe_unused]] static __global__ void __launch_bounds__(kBlock) msda_zero_kernel(uint4* __restrict__ p, int64_t n16) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Round the float32 accumulator to fp16/bf16 (nearest even), 8 elements per
// lane per step (n8 = element count / 8).
template <int DT>
__global__ void __launch_bounds__(kBlock)
msda_narrow_kernel(const float4* __restrict__ src, uint4* __restrict__ dst, int64_t n8) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n8; i += stride) {
        float4 a = src[2 * i], c = src[2 * i + 1];
        float f[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        Raw<16> r = narrow<DT, 16>(f);
        dst[i] = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
    }
}

__device__ __forceinline__ void atomic_add_f32(float* p, float v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Float add into LDS through an integer compare-and-swap loop (LDS integer
// atomics are far faster than ds_add_f32 on gfx950).
__device__ __forceinline__ void lds_add_f32(float* p, float v) {
    uint32_t* u = reinterpret_cast<uint32_t*>(p);
    uint32_t old = __hip_atomic_load(u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (true) {
        uint32_t expect = old;
        const uint32_t want = __float_as_uint(__uint_as_float(old) + v);
        if (__hip_atomic_compare_exchange_strong(u, &expect, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP))
            break;
        old = expect;
    }
}

// dst[0..N) += v[0..N) in LDS.  For even N (dst 8-byte aligned): N/2 64-bit
// compare-and-swaps per round, all issued before any result is checked; a
// pair already added re-swaps the value it last saw with itself, which
// changes nothing.  Odd N falls back to one 32-bit loop per float.
template <int N>
__device__ __forceinline__ void lds_add_f32xN(float* dst, const float* v) {
    if constexpr (N % 2 != 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) lds_add_f32(dst + i, v[i]);
    } else {
        constexpr int NP = N / 2;
        uint64_t* u = reinterpret_cast<uint64_t*>(dst);
        uint64_t seen[NP];
        bool done[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            seen[i] = __hip_atomic_load(u + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            done[i] = false;
        }
        bool all;
        do {
            all = true;
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const float lo = __uint_as_float(static_cast<uint32_t>(seen[i])) + v[2 * i];
                const float hi = __uint_as_float(static_cast<uint32_t>(seen[i] >> 32)) + v[2 * i + 1];
                const uint64_t sum = static_cast<uint64_t>(__float_as_uint(lo)) |
                                     (static_cast<uint64_t>(__float_as_uint(hi)) << 32);
                uint64_t expect = seen[i];
                const bool ok = __hip_atomic_compare_exchange_strong(u + i, &expect, done[i] ? seen[i] : sum,
                                                                     __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                                     __HIP_MEMORY_SCOPE_WORKGROUP);
                if (!done[i]) seen[i] = expect;
                done[i] = done[i] || ok;
                all = all && done[i];
            }
        } while (!all);
    }
}

// ---------------------------------------------------------------------------
// 1. count
// ---------------------------------------------------------------------------
// Samples [s_begin, s_end) of plane (b, m), in the plane's (query, level,
// point) order, counted into the LDS histogram `hist` (nseg bins), NT lanes.
// REF as for the gradient kernel (loc holds the offsets and ref the reference
// points when REF != 0).  s_lv: the staged level table.
template <int DT, int L_CT, int P_CT, int REF, int NT>
__device__ __forceinline__ void count_samples(const void* __restrict__ loc, const void* __restrict__ ref,
                                              int32_t* hist, const int4* s_lv, const Problem& pb, int b, int m,
                                              int s_begin, int s_end) {
    const int L = L_CT ? L_CT : pb.L;
    const int P = P_CT ? P_CT : pb.P;
    const int LP = L * P;
    // S samples per location load (one 16-byte load of S consecutive samples
    // of a group, as in the gradient kernel's prologue); s_begin and s_end are
    // multiples of S then
    constexpr int S = kPrologueSamples<sample_dt(DT), REF, L_CT, P_CT>;
    constexpr int SE = Elem<sample_dt(DT)>::bytes;
    constexpr int kU = 4;                            // loads in flight together
    for (int s0 = s_begin + S * static_cast<int>(threadIdx.x); s0 < s_end; s0 += kU * S * NT) {
        float lx[kU * S], ly[kU * S];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int s = s0 + u * S * NT;
#pragma unroll
            for (int k = 0; k < S; ++k) lx[u * S + k] = ly[u * S + k] = -2.0f;   // off the map
            if (s < s_end) {
                const int q = s / LP, lp = s - q * LP, l = lp / P;
                const int64_t i = ((static_cast<int64_t>(b) * pb.Q + q) * pb.M + m) * LP + lp;
                if constexpr (S > 1) {
                    float xy[2 * S];
                    widen<sample_dt(DT), 16>(load_raw<16>(static_cast<const char*>(loc) + 2 * i * SE), xy);
#pragma unroll
                    for (int k = 0; k < S; ++k) {
                        lx[u * S + k] = xy[2 * k];
                        ly[u * S + k] = xy[2 * k + 1];
                    }
                } else {
                    const int64_t ri = (static_cast<int64_t>(b) * pb.Q + q) * L + l;
                    const int4 lv = s_lv[l];
                    const float2 xy = sample_location<sample_dt(DT), REF>(loc, ref, i, ri, static_cast<float>(lv.y),
                                                                           static_cast<float>(lv.x),
                                                                           static_cast<float>(P));
                    lx[u] = xy.x;
                    ly[u] = xy.y;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            // the cells of the S samples (kNoCell off the map or past the end)
            uint32_t cell[S];
#pragma unroll
            for (int k = 0; k < S; ++k) {
                const int s = s0 + u * S * NT + k;
                const int4 lv = s_lv[(s % LP) / P];
                float x, y;
                cell[k] = s < s_end && pixel_coords(lx[u * S + k], ly[u * S + k], static_cast<float>(lv.y),
                                                    static_cast<float>(lv.x), x, y)
                              ? pack_cell(static_cast<int>(floorf(x)), static_cast<int>(floorf(y)))
                              : kNoCell;
            }
            // merged records count once (a lane pair's samples are valid
            // together: s_begin and s_end are multiples of four)
            uint32_t rows[S];
#pragma unroll
            for (int k = 0; k < S; ++k) rows[k] = 3u;
            if constexpr (kMergeRecords<REF, L_CT, P_CT>)
                if (pb.merge_records) record_rows<S>(cell, (s0 + u * S * NT) % P, rows);
#pragma unroll
            for (int k = 0; k < S; ++k) {
                if (cell[k] == kNoCell) continue;
                const int4 lv = s_lv[((s0 + u * S * NT + k) % LP) / P];
                const int x0 = static_cast<int>(cell[k] & 0xffffu) - 1, y0 = static_cast<int>(cell[k] >> 16) - 1;
                for_each_record(
                    x0, y0, lv.y, lv.x, lv.w & 0xff, lv.w >> 8,
                    [&](int seg, int, int, int) { atomicAdd(&hist[seg], 1); }, rows[k]);
            }
        }
    }
}

// Grid: nplanes * nchunks workgroups of kCountBlock lanes, chunk samples
// each (the last chunk of a plane may be short).  Each workgroup writes its
// own histogram row counts[(plane * nchunks + chunk) * nseg ...] in full, so
// no buffer needs zeroing first.  LDS: nseg int32.
template <int DTK, int L_CT, int P_CT, int REF>
__global__ void __launch_bounds__(kCountBlock)
msda_bin_count_kernel(const void* __restrict__ loc, const void* __restrict__ ref, int32_t* __restrict__ counts,
                      Problem pb, int chunk) {
    extern __shared__ int32_t hist[];
    const int LP = (L_CT ? L_CT : pb.L) * (P_CT ? P_CT : pb.P);
    const int nsamp = pb.Q * LP;
    const int nchunks = (nsamp + chunk - 1) / chunk;
    const int pl = blockIdx.x / nchunks, c = blockIdx.x - pl * nchunks;
    const int b = pl / pb.M, m = pl - b * pb.M;

    __shared__ int4 s_lv[kMaxLevels];
    stage_levels(pb, s_lv);
    for (int i = threadIdx.x; i < pb.nseg; i += kCountBlock) hist[i] = 0;
    __syncthreads();
    count_samples<DTK, L_CT, P_CT, REF, kCountBlock>(loc, ref, hist, s_lv, pb, b, m, c * chunk,
                                                    min((c + 1) * chunk, nsamp));
    __syncthreads();
    int32_t* row = counts + static_cast<int64_t>(blockIdx.x) * pb.nseg;
    for (int i = threadIdx.x; i < pb.nseg; i += kCountBlock) row[i] = hist[i];
}

// ---------------------------------------------------------------------------
// 2. scan
// ---------------------------------------------------------------------------

__device__ __forceinline__ int units_of(int count, int unit) {
    return count <= unit ? 1 : (count + unit - 1) / unit;
}

// Zero the float32 rows of plane-global segment `gs`, lanes t, t+nt, ...
__device__ void zero_segment(const Problem& pb, float* gacc, int gs, int t, int nt) {
    const int pl = gs / pb.nseg, seg = gs - pl * pb.nseg;
    const int b = pl / pb.M, m = pl - b * pb.M;
    const int l = level_of_segment(pb, seg);
    const int k0 = (seg - pb.seg_base[l]) << pb.seg_shift[l];
    const int nk = min(1 << pb.seg_shift[l], pb.lv.H[l] * pb.lv.W[l] - k0);
    const int d4 = pb.D / 4;                          // 16-byte stores (D is a multiple of 8)
    const UDiv by_d4 = udiv_by(d4);                   // (i < nk * d4 <= 2^14)
    for (int i = t; i < nk * d4; i += nt) {
        const int k = udiv(i, by_d4), c = i - k * d4;
        const int64_t key = pb.lv.start[l] + k0 + k;
        *reinterpret_cast<float4*>(gacc + ((static_cast<int64_t>(b) * pb.K + key) * pb.M + m) * pb.D + 4 * c) =
            make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
}

// Round the float32 rows of plane-global segment `gs` to dtype DT into
// `out`, 8 elements per lane step, lanes t, t+nt, ...
template <int DT>
__device__ void narrow_segment(const Problem& pb, const float* gacc, void* out, int gs, int t, int nt) {
    const int pl = gs / pb.nseg, seg = gs - pl * pb.nseg;
    const int b = pl / pb.M, m = pl - b * pb.M;
    const int l = level_of_segment(pb, seg);
    const int k0 = (seg - pb.seg_base[l]) << pb.seg_shift[l];
    const int nk = min(1 << pb.seg_shift[l], pb.lv.H[l] * pb.lv.W[l] - k0);
    const int d8 = pb.D / 8;
    const UDiv by_d8 = udiv_by(d8);                   // (i < nk * d8 <= 2^13)
    for (int i = t; i < nk * d8; i += nt) {
        const int k = udiv(i, by_d8), c = i - k * d8;
        const int64_t e = ((static_cast<int64_t>(b) * pb.K + pb.lv.start[l] + k0 + k) * pb.M + m) * pb.D + 8 * c;
        const float4 a = *reinterpret_cast<const float4*>(gacc + e);
        const float4 z = *reinterpret_cast<const float4*>(gacc + e + 4);
        const float f[8] = {a.x, a.y, a.z, a.w, z.x, z.y, z.z, z.w};
        const Raw<16> r = narrow<DT, 16>(f);
        *reinterpret_cast<uint4*>(static_cast<char*>(out) + e * 2) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
    }
}

// 16-bit dtypes: the rows of the segments split over several units (the
// only rows the accumulation leaves in the float32 workspace), rounded into
// grad_value.  Grid: nplanes * kNarrowPerPlane workgroups.

template <int DT>
__global__ void __launch_bounds__(kBlock)
msda_narrow_segments_kernel(const float* __restrict__ gacc, void* __restrict__ out,
                            const int32_t* __restrict__ nunits, const int32_t* __restrict__ multi, Problem pb) {
    const int pl = blockIdx.x / kNarrowPerPlane, sub = blockIdx.x - pl * kNarrowPerPlane;
    const int nm = nunits[pb.nplanes + pl];
    for (int e = sub; e < nm; e += kNarrowPerPlane)
        narrow_segment<DT>(pb, gacc, out, multi[static_cast<int64_t>(pl) * pb.nseg + e], threadIdx.x, kBlock);
}

// Plane p owns a fixed record region [p * plane_records, ...) and a fixed
// unit region [p * plane_units, ...), so planes need no common prefix.  From
// the plane's segment counts (LDS s_cnt), NT lanes write: the cursors (the
// exclusive prefix plus the region base), the plane's units {segment, first
// record, end record, flush-with-atomics} and their number (nunits[p]), and
// the plane's segments split over several units (nunits[nplanes + p]
// entries of multi[p * nseg ...]), whose rows the gradient kernel zeroes.
// With `accumulate` every unit adds into the caller's buffer, which is then
// left as it is (and no segment is listed).  Every lane scans kMaxSegments /
// NT consecutive segments; lanes combine through a wave scan and the wave
// totals.  Ends with a barrier; s_nmulti must be zero on entry.
template <int NT>
__device__ void scan_plane(const int32_t* s_cnt, int32_t* s_wrec, int32_t* s_wunit, int32_t* s_nmulti,
                           int32_t* __restrict__ cursor, int32_t* __restrict__ nunits,
                           int32_t* __restrict__ multi, int4* __restrict__ units, int accumulate,
                           const Problem& pb, int pl, int plane_records, int plane_units) {
    constexpr int kPer = kMaxSegments / NT;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int n = pb.nseg;
    const int64_t cbase = static_cast<int64_t>(pl) * n;
    int rsum = 0, usum = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = t * kPer + j;
        if (i < n) {
            rsum += s_cnt[i];
            usum += units_of(s_cnt[i], pb.unit_records);
        }
    }
    int rinc = rsum, uinc = usum;                    // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int ru = __shfl_up(rinc, o, 64), uu = __shfl_up(uinc, o, 64);
        if (lane >= o) {
            rinc += ru;
            uinc += uu;
        }
    }
    if (lane == 63) {
        s_wrec[wave] = rinc;
        s_wunit[wave] = uinc;
    }
    __syncthreads();
    int rbase = rinc - rsum, ubase = uinc - usum;
    for (int w = 0; w < wave; ++w) {
        rbase += s_wrec[w];
        ubase += s_wunit[w];
    }
    rbase += pl * plane_records;
    const int ufirst = pl * plane_units;
#pragma unroll 1
    for (int j = 0; j < kPer; ++j) {
        const int i = t * kPer + j;
        if (i >= n) break;
        const int c = s_cnt[i], u = units_of(c, pb.unit_records);
        const int gi = static_cast<int>(cbase) + i;
        cursor[gi] = rbase;
        const int atomic_flush = (u > 1 || accumulate) ? 1 : 0;
        for (int k = 0; k < u; ++k)
            units[ufirst + ubase + k] = make_int4(gi, rbase + k * pb.unit_records,
                                                  rbase + min(c, (k + 1) * pb.unit_records), atomic_flush);
        if (u > 1 && !accumulate) multi[cbase + atomicAdd(s_nmulti, 1)] = gi;
        rbase += c;
        ubase += u;
    }
    __syncthreads();
    if (t == NT - 1) {
        nunits[pl] = ubase;                          // the last lane's running count is the total
        nunits[pb.nplanes + pl] = *s_nmulti;
    }
}

// One workgroup of kScanBlock lanes per plane: sums the plane's nchunks
// histogram rows, then scan_plane.  Up to four lanes share a segment's rows
// (every parts-th row each, combined by lane shuffles), so that a segment's
// loads are spread over several lanes.  (static: every translation unit that
// launches it has its own copy, as for the other non-template kernels.)
constexpr int kScanBlock = 1024;

[[maybe_unused]] static __global__ void __launch_bounds__(kScanBlock)
msda_bin_scan_kernel(const int32_t* __restrict__ counts, int nchunks, int32_t* __restrict__ cursor,
                     int32_t* __restrict__ nunits, int32_t* __restrict__ multi, int4* __restrict__ units,
                     int accumulate, Problem pb, int plane_records, int plane_units) {
    __shared__ int32_t s_cnt[kMaxSegments];
    __shared__ int32_t s_wrec[kScanBlock / 64], s_wunit[kScanBlock / 64];
    __shared__ int32_t s_nmulti;
    __shared__ unsigned long long s_total;
    const int pl = blockIdx.x, n = pb.nseg;
    if (threadIdx.x == 0) {
        s_nmulti = 0;
        s_total = 0;
    }
    __syncthreads();
    const int32_t* rows = counts + static_cast<int64_t>(pl) * nchunks * n;
    // lanes per segment: 4, 2 or 1, as many as the workgroup holds; a
    // segment's lanes are adjacent (same wave, same trip count)
    const int parts = 4 * n <= kScanBlock ? 4 : (2 * n <= kScanBlock ? 2 : 1);
    const int t = static_cast<int>(threadIdx.x), part = t % parts;
    for (int i = t / parts; i < n; i += kScanBlock / parts) {
        int sum = 0;
#pragma unroll 8
        for (int c = part; c < nchunks; c += parts) sum += rows[static_cast<int64_t>(c) * n + i];
        if (parts >= 2) sum += __shfl_xor(sum, 1, 64);
        if (parts >= 4) sum += __shfl_xor(sum, 2, 64);
        if (part == 0) {
            // rows that a counting forward left are trusted only as far as
            // they fit the plane's fixed regions (see below)
            sum = min(max(sum, 0), plane_records);
            s_cnt[i] = sum;
            atomicAdd(&s_total, static_cast<unsigned long long>(sum));
        }
    }
    __syncthreads();
    // Counts that exceed the plane's record region cannot come from the
    // plane's own samples (a counting forward on other locations, or rows
    // never written): they are dropped, so that every cursor and unit stays
    // within the plane's regions.  The backward's results are then wrong,
    // but no access leaves the workspace.
    if (s_total > static_cast<unsigned long long>(plane_records)) {
        for (int i = threadIdx.x; i < n; i += kScanBlock) s_cnt[i] = 0;
        __syncthreads();
    }
    scan_plane<kScanBlock>(s_cnt, s_wrec, s_wunit, &s_nmulti, cursor, nunits, multi, units, accumulate, pb, pl,
                           plane_records, plane_units);
}

// Count and scan in one launch, one workgroup of kCountScanBlock lanes per
// plane, for planes of at most kCountScanSamples samples (a latency-bound
// size: one launch and no histogram rows in memory).
constexpr int kCountScanBlock = 1024;

template <int DTK, int L_CT, int P_CT, int REF>
__global__ void __launch_bounds__(kCountScanBlock)
msda_bin_count_scan_kernel(const void* __restrict__ loc, const void* __restrict__ ref,
                           int32_t* __restrict__ cursor, int32_t* __restrict__ nunits, int32_t* __restrict__ multi,
                           int4* __restrict__ units, int accumulate, Problem pb, int plane_records,
                           int plane_units) {
    __shared__ int32_t s_cnt[kMaxSegments];
    __shared__ int32_t s_wrec[kCountScanBlock / 64], s_wunit[kCountScanBlock / 64];
    __shared__ int32_t s_nmulti;
    __shared__ int4 s_lv[kMaxLevels];
    const int pl = blockIdx.x;
    const int b = pl / pb.M, m = pl - b * pb.M;
    const int LP = (L_CT ? L_CT : pb.L) * (P_CT ? P_CT : pb.P);
    stage_levels(pb, s_lv);
    if (threadIdx.x == 0) s_nmulti = 0;
    for (int i = threadIdx.x; i < pb.nseg; i += kCountScanBlock) s_cnt[i] = 0;
    __syncthreads();
    count_samples<DTK, L_CT, P_CT, REF, kCountScanBlock>(loc, ref, s_cnt, s_lv, pb, b, m, 0, pb.Q * LP);
    __syncthreads();
    scan_plane<kCountScanBlock>(s_cnt, s_wrec, s_wunit, &s_nmulti, cursor, nunits, multi, units, accumulate, pb,
                                pl, plane_records, plane_units);
}

// ---------------------------------------------------------------------------
// 3a. float-atomic grad_value with a workgroup pre-reduction
// ---------------------------------------------------------------------------
// Outside the record envelope the gradient workgroup adds its grad_value
// contributions into float32 rows with global atomics.  Adding every sample
// corner on its own makes a row that many samples reach (a coarse level) the
// float32 sum of thousands of atomic adds in arbitrary order, whose rounding
// can exceed the float32 bar.  So the workgroup first merges its corners by
// row: every in-map corner of its samples is an entry (sample * 4 + corner,
// 16 bits), counting-sorted into kPreBuckets buckets by a hash of the row;
// one worker (LPR lanes) walks a bucket, summing the contributions
// w * (bilinear weight) * grad_output of consecutive entries of one row in
// registers, and adds each run once.  Rows that share a bucket interleave
// there, which only splits their runs.  No LDS float atomics (slow on
// gfx950): the sort uses integer ones.  A row reached by n corners of the
// workgroup gets one atomic add per element instead of n.
constexpr int kPreBuckets = 1024;

__device__ __forceinline__ int pre_bucket(uint32_t off) { return static_cast<int>((off * 0x9E3779B1u) >> 22); }

// srec: the prologue's sample records (8 words each: the four corner byte
// offsets, lx, ly, the attention weight, the cell); pre_g: the workgroup's
// grad_output rows as float32; gplane: the float32 rows of the workgroup's
// (batch, head) plane, element offset = corner byte offset / E.  Starts
// after a barrier; every lane of the workgroup calls it.
template <int DT, int VECB, int LPR>
__device__ void pre_reduce_scatter(const uint32_t* srec, int gstride, int LP, int gcount, const float* pre_g,
                                   int32_t* start, int32_t* end, uint16_t* ids, float* gplane, const Problem& pb) {
    constexpr int E = Elem<DT>::bytes;
    constexpr int VEC = VECB / E;
    const int nt = blockDim.x, ns = gcount * LP;
    for (int i = threadIdx.x; i < kPreBuckets; i += nt) end[i] = 0;
    __syncthreads();
    for (int s = threadIdx.x; s < ns; s += nt) {
        const uint4 o = *reinterpret_cast<const uint4*>(srec + (s / LP) * gstride + (s % LP) * 8);
        if (o.x != kOffMap) atomicAdd(&end[pre_bucket(o.x)], 1);
        if (o.y != kOffMap) atomicAdd(&end[pre_bucket(o.y)], 1);
        if (o.z != kOffMap) atomicAdd(&end[pre_bucket(o.z)], 1);
        if (o.w != kOffMap) atomicAdd(&end[pre_bucket(o.w)], 1);
    }
    __syncthreads();
    if (threadIdx.x < 64) {                          // exclusive scan of the counts, one wave
        constexpr int kPer = kPreBuckets / 64;
        const int lane = threadIdx.x;
        int sum = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) sum += end[lane * kPer + j];
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int up = __shfl_up(incl, o, 64);
            if (lane >= o) incl += up;
        }
        int run = incl - sum;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int c = end[lane * kPer + j];
            start[lane * kPer + j] = run;
            end[lane * kPer + j] = run;              // the cursor; the bucket's end once filled
            run += c;
        }
    }
    __syncthreads();
    for (int s = threadIdx.x; s < ns; s += nt) {
        const uint4 o = *reinterpret_cast<const uint4*>(srec + (s / LP) * gstride + (s % LP) * 8);
        const uint32_t oc[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (oc[c] != kOffMap) ids[atomicAdd(&end[pre_bucket(oc[c])], 1)] = static_cast<uint16_t>(4 * s + c);
    }
    __syncthreads();
    const int nw = nt / LPR, w = threadIdx.x / LPR, li = threadIdx.x % LPR;
    const bool active = li < pb.lpr_active;
    float* dst = gplane + li * VEC;
    for (int bk = w; bk < kPreBuckets; bk += nw) {
        const int e1 = end[bk];
        uint32_t row = kOffMap;
        float acc[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
        for (int e = start[bk]; e < e1; ++e) {
            const int id = ids[e], s = id >> 2, c = id & 3, g = s / LP;
            const uint32_t* r = srec + g * gstride + (s - g * LP) * 8;
            const uint32_t off = r[c];
            const float lx = fabsf(__uint_as_float(r[4])), ly = fabsf(__uint_as_float(r[5])), aw = __uint_as_float(r[6]);
            // the corner's weight: w * (1-ly or ly) * (1-lx or lx)
            const float wy = aw * ((c & 2) ? ly : 1.0f - ly);
            const float cw = wy * ((c & 1) ? lx : 1.0f - lx);
            if (off != row) {
                if (row != kOffMap && active) {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) atomic_add_f32(dst + row / E + i, acc[i]);
                }
                row = off;
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
            }
            const float* gg = pre_g + g * pb.D + li * VEC;
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] += cw * gg[i];
        }
        if (row != kOffMap && active) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) atomic_add_f32(dst + row / E + i, acc[i]);
        }
    }
}

// ---------------------------------------------------------------------------
// 3. gradient (gather): grad_w, grad_loc, and grad_value records or atomics
// ---------------------------------------------------------------------------
// Grid: nplanes * ceil(Q / gpb) workgroups of gpb * LPR lanes, plane-local
// as in the forward.  A prologue (one lane per sample) stores each sample's
// corner offsets, fractions lx, ly, attention weight and packed cell
// (x0 + 1, y0 + 1) in LDS (8 words; hx, hy and the weight products are
// recomputed from them with the same roundings) and counts its records per
// segment; the main loop gathers the four corner rows of each sample, forms
// the four dot products with the query's grad_output row and reduces them
// over the group's lanes; when BINNED, an epilogue reserves the workgroup's
// record ranges, writes the records, and has the plane's workgroups zero the
// rows of the plane's multi-unit segments (the accumulation adds into them).
// LDS: gpb * (8 * L * P + 4) words; when BINNED also 2 * nseg int32 (counts,
// then cursors, and bases); otherwise the pre-reduction's gpb * D floats,
// 2 * kPreBuckets int32 and 4 * gpb * L * P uint16 (pre_reduce_scatter).
template <int DTK, int VECB, int LPR, int L_CT, int P_CT, bool BINNED, int REF>
__global__ void __launch_bounds__(kBlock)
msda_backward_kernel(const void* __restrict__ value, const void* __restrict__ loc,
                     const void* __restrict__ attw, const void* __restrict__ ref,
                     const uint8_t* __restrict__ kmask, const void* __restrict__ gout,
                     float* __restrict__ gacc, uint3* __restrict__ recs, int32_t* __restrict__ cursor,
                     int32_t* __restrict__ nunits, const int32_t* __restrict__ multi,
                     void* __restrict__ grad_loc, void* __restrict__ grad_w, Problem pb, int gpb) {
    constexpr int DT = value_dt(DTK), ST = sample_dt(DTK);
    constexpr int E = Elem<DT>::bytes;
    constexpr int VEC = VECB / E;
    constexpr bool kFixedLP = L_CT != 0 && P_CT != 0;
    const int L = L_CT ? L_CT : pb.L;
    const int P = P_CT ? P_CT : pb.P;
    const int LP = L * P;
    const int gstride = 8 * LP + 4;

    extern __shared__ uint32_t sm[];
    uint32_t* srec = sm;
    int32_t* lhist = reinterpret_cast<int32_t*>(sm + gpb * gstride);
    int32_t* lbase = lhist + pb.nseg;
    // fused prologue: logits (later the weights' gradients) and exponentials
    float* sv = reinterpret_cast<float*>(lhist + (BINNED ? 2 * pb.nseg : 0));
    float* se = sv + gpb * LP;
    // float-atomic path: the workgroup's grad_output rows (gpb * D floats),
    // bucket starts and ends (kPreBuckets int32 each), entry ids (4 * gpb * LP u16)
    float* pre_g = REF != 0 ? se + gpb * LP : sv;
    int32_t* pre_start = reinterpret_cast<int32_t*>(pre_g + gpb * pb.D);
    int32_t* pre_end = pre_start + kPreBuckets;
    uint16_t* pre_id = reinterpret_cast<uint16_t*>(pre_end + kPreBuckets);

    const PlaneTile t = plane_tile(pb, gpb);
    const uint32_t pitch = static_cast<uint32_t>(pb.M * pb.D * E);
    __shared__ int4 s_lv[kMaxLevels];
    stage_levels(pb, s_lv);
    if constexpr (BINNED)
        for (int i = threadIdx.x; i < pb.nseg; i += blockDim.x) lhist[i] = 0;
    if constexpr (REF != 0) load_logits<ST>(attw, t.G0, pb.M, t.gcount, LP, sv);
    __syncthreads();
    if constexpr (REF != 0) {
        exp_logits(t.gcount, LP, sv, se);
        __syncthreads();
    }

    // prologue: sample i = g * LP + lp of the workgroup, its corners c (from
    // its location) and (REF == 0) its attention weight w_in -> LDS record and
    // segment counts (of its records on the image rows in `rows`, bit r for
    // row y0 + r: all, or those record merging leaves it).
    // With REF != 0 the weight kept is the softmax weight even for a sample
    // off the map (its gradient reaches the other logits of the group);
    // nothing reads it there but the softmax backward.
    auto corners_of = [&](int lp, float2 xy) {
        const int4 lv = s_lv[lp / P];
        Corners c = sample_corners(xy.x, xy.y, lv.x, lv.y, lv.z, pitch);
        // padded corners read as zero; their records still go to the
        // accumulation, which writes padded rows as zero
        mask_corners(c, kmask ? kmask + static_cast<int64_t>(t.b) * pb.K : nullptr, lv.z, lv.y);
        return c;
    };
    auto stage = [&](int i, int g, int lp, const Corners& c, float w_in, uint32_t rows) {
        const int4 lv = s_lv[lp / P];
        const int H = lv.x, W = lv.y;
        float aw;
        if constexpr (REF == 0) aw = c.ok ? w_in : 0.0f;
        else aw = se[i] / group_total(se + g * LP, LP);
        uint32_t* r = srec + g * gstride + lp * 8;
        const uint32_t cell = c.ok ? pack_cell(c.x0, c.y0) : kNoCell;
        // record merging: a row whose record another point makes is marked
        // by the sign bit of lx (row y0) or ly (row y0 + 1), which are never
        // negative otherwise (readers take their magnitudes)
        const uint32_t drop0 = c.ok && (rows & 1u) == 0u ? 0x80000000u : 0u;
        const uint32_t drop1 = c.ok && (rows & 2u) == 0u ? 0x80000000u : 0u;
        *reinterpret_cast<uint4*>(r) = make_uint4(c.o00, c.o01, c.o10, c.o11);
        *reinterpret_cast<uint4*>(r + 4) = make_uint4(__float_as_uint(c.lx) | drop0, __float_as_uint(c.ly) | drop1,
                                                      __float_as_uint(aw), cell);
        if constexpr (BINNED) {
            if (c.ok)
                for_each_record(
                    c.x0, c.y0, W, H, lv.w & 0xff, lv.w >> 8,
                    [&](int seg, int, int, int) { atomicAdd(&lhist[seg], 1); }, rows);
        }
    };
    if constexpr (kPrologueSamples<ST, REF, L_CT, P_CT> > 1) {
        // S samples of one group per lane: their locations in one 16-byte
        // load, their weights in one 8-byte load (fewer load instructions
        // through the texture path the main loop saturates)
        constexpr int S = kPrologueSamples<ST, REF, L_CT, P_CT>;
        constexpr int SE = Elem<ST>::bytes;
        for (int i = S * threadIdx.x; i < t.gcount * LP; i += S * blockDim.x) {
            const int g = i / LP, lp = i - g * LP;
            const int64_t si = (t.G0 + static_cast<int64_t>(g) * pb.M) * LP + lp;
            float xy[2 * S], wv[S];
            widen<ST, 16>(load_raw<16>(static_cast<const char*>(loc) + 2 * si * SE), xy);
            widen<ST, S * SE>(load_raw<S * SE>(static_cast<const char*>(attw) + si * SE), wv);
            Corners c[S];
            uint32_t rows[S];
#pragma unroll
            for (int k = 0; k < S; ++k) {
                c[k] = corners_of(lp + k, make_float2(xy[2 * k], xy[2 * k + 1]));
                rows[k] = 3u;
            }
            if constexpr (BINNED && kMergeRecords<REF, L_CT, P_CT>) {
                if (pb.merge_records) {
                    // (the lane pair holding a level's four points is active
                    // together: t.gcount * LP and the loop stride are multiples
                    // of four)
                    uint32_t cell[S];
#pragma unroll
                    for (int k = 0; k < S; ++k) cell[k] = c[k].ok ? pack_cell(c[k].x0, c[k].y0) : kNoCell;
                    record_rows<S>(cell, lp % P, rows);
                }
            }
#pragma unroll
            for (int k = 0; k < S; ++k) stage(i + k, g, lp + k, c[k], wv[k], rows[k]);
        }
    } else {
        for (int i = threadIdx.x; i < t.gcount * LP; i += blockDim.x) {
            const int g = i / LP, lp = i - g * LP, l = lp / P;
            const int64_t si = (t.G0 + static_cast<int64_t>(g) * pb.M) * LP + lp;
            const int4 lv = s_lv[l];
            const int64_t ri = (static_cast<int64_t>(t.b) * pb.Q + t.q0 + g) * L + l;
            const float2 xy = sample_location<ST, REF>(loc, ref, si, ri, static_cast<float>(lv.y),
                                                       static_cast<float>(lv.x), static_cast<float>(P));
            float w_in = 0.0f;
            if constexpr (REF == 0) w_in = load_scalar<ST>(attw, si);
            stage(i, g, lp, corners_of(lp, xy), w_in, 3u);
        }
    }
    __syncthreads();

    const int lg = threadIdx.x / LPR, li = threadIdx.x % LPR;
    if (lg < t.gcount) {
        const bool active = li < pb.lpr_active;
        const int64_t G = t.G0 + static_cast<int64_t>(lg) * pb.M;
        const __amdgpu_buffer_rsrc_t vr = value_plane<E>(value, pb, t.b, t.m);
        // lanes past the row read zeros through an off-map offset
        const uint32_t lane_b = active ? static_cast<uint32_t>(li * VECB) : kOffMap;
        const uint32_t* rec = srec + lg * gstride;

        // the query's grad_output row: packed (16-bit dtypes, for the dot2
        // products below) and widened
        Raw<VECB> graw;
#pragma unroll
        for (int i = 0; i < VECB / 4; ++i) graw.w[i] = 0u;
        if (active) graw = load_raw<VECB>(static_cast<const char*>(gout) + (G * pb.D + li * VEC) * E);
        float g[VEC];
        widen<DT, VECB>(graw, g);
        if constexpr (!BINNED) {
            // the query's grad_output row, for the pre-reduction below
            if (active) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) pre_g[lg * pb.D + li * VEC + i] = g[i];
            }
        }
        // Samples go in chunks of kC (LPR, or all of them when fewer): lane li
        // of the group keeps the results of the chunk's sample li and stores
        // them after the chunk, so a group's stores are contiguous.  Within a
        // chunk, kSB samples' corner loads are in flight together.
        constexpr int kC = kFixedLP ? (LPR < L_CT * P_CT ? LPR : L_CT * P_CT) : 1;
        // (two for float32, whose occupancy then doubles; four for 16-bit rows)
        constexpr int kSBMax = E == 4 ? 2 : 4;
        constexpr int kSB = kC % kSBMax == 0 ? kSBMax : 1;
        // Plain form with L * P = kOwn * LPR, kOwn dividing LPR and kOwn
        // weights filling 8 or 16 bytes: lane li keeps the results of samples
        // kOwn * li .. kOwn * li + kOwn - 1 over all chunks and stores them
        // once, grad_loc in one or two 16-byte stores and grad_w in one.
        constexpr int kOwnLP = kFixedLP ? (L_CT * P_CT) / LPR : 0;
        constexpr int kOwn = REF == 0 && kFixedLP && (L_CT * P_CT) % LPR == 0 && kOwnLP > 1 &&
                                     LPR % kOwnLP == 0 &&
                                     (kOwnLP * Elem<ST>::bytes == 8 || kOwnLP * Elem<ST>::bytes == 16)
                                 ? kOwnLP
                                 : 1;
        float keep_w[kOwn], keep_x[kOwn], keep_y[kOwn];
#pragma unroll
        for (int k = 0; k < kOwn; ++k) keep_w[k] = keep_x[k] = keep_y[k] = 0.0f;
#pragma unroll 1
        for (int c0 = 0; c0 < LP; c0 += kC) {
            float own_w = 0.0f, own_x = 0.0f, own_y = 0.0f;
            int own_l = 0;                                   // level of the owned sample
#pragma unroll
            for (int b0 = 0; b0 < kC; b0 += kSB) {
                uint4 o[kSB];
                Raw<VECB> raw[kSB][4];
#pragma unroll
                for (int u = 0; u < kSB; ++u) {
                    o[u] = *reinterpret_cast<const uint4*>(rec + (c0 + b0 + u) * 8);
                    raw[u][0] = buffer_load<VECB>(vr, o[u].x + lane_b);
                    raw[u][1] = buffer_load<VECB>(vr, o[u].y + lane_b);
                    raw[u][2] = buffer_load<VECB>(vr, o[u].z + lane_b);
                    raw[u][3] = buffer_load<VECB>(vr, o[u].w + lane_b);
                }
                // a batch of several samples: its loads all go out before
                // the first use (left to itself the scheduler issues them one
                // at a time; encoder gradient 131 -> 129 us, large-batch bf16
                // 462 -> 455 us)
                if constexpr (kSB > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < kSB; ++u) {
                    const int lp = c0 + b0 + u;
                    const float4 fr = *reinterpret_cast<const float4*>(rec + lp * 8 + 4);    // lx ly w cell
                    const float flx = fabsf(fr.x), fly = fabsf(fr.y);                        // (sign: merging)
                    const float4 f = make_float4(1.0f - flx, flx, 1.0f - fly, fly);          // hx lx hy ly
                    float d00 = 0.0f, d01 = 0.0f, d10 = 0.0f, d11 = 0.0f;
                    if constexpr (DT == kF32) {
                        float v00[VEC], v01[VEC], v10[VEC], v11[VEC];
                        widen<DT, VECB>(raw[u][0], v00);
                        widen<DT, VECB>(raw[u][1], v01);
                        widen<DT, VECB>(raw[u][2], v10);
                        widen<DT, VECB>(raw[u][3], v11);
#pragma unroll
                        for (int i = 0; i < VEC; ++i) {
                            d00 += g[i] * v00[i];
                            d01 += g[i] * v01[i];
                            d10 += g[i] * v10[i];
                            d11 += g[i] * v11[i];
                        }
                    } else {
                        // 16-bit rows: <g, v> two elements per instruction
                        // (v_dot2_f32_{f16,bf16}: exact products, float32
                        // sums), straight from the packed rows
#pragma unroll
                        for (int i = 0; i < VECB / 4; ++i) {
                            d00 = dot2<DT>(raw[u][0].w[i], graw.w[i], d00);
                            d01 = dot2<DT>(raw[u][1].w[i], graw.w[i], d01);
                            d10 = dot2<DT>(raw[u][2].w[i], graw.w[i], d10);
                            d11 = dot2<DT>(raw[u][3].w[i], graw.w[i], d11);
                        }
                    }
                    const float top = f.x * d00 + f.y * d01;
                    const float bot = f.x * d10 + f.y * d11;
                    const float sw = group_sum<LPR>(f.z * top + f.w * bot);
                    const float sx = group_sum<LPR>(f.z * (d01 - d00) + f.w * (d11 - d10));
                    const float sy = group_sum<LPR>(bot - top);
                    // a sample off the map (all four corners at kOffMap) gets exactly
                    // zero gradients, whatever grad_output holds
                    const bool off = ((o[u].x & o[u].y & o[u].z & o[u].w) & kOffMap) != 0u;
                    if constexpr (kOwn > 1) {
                        // chunks start at multiples of LPR, a multiple of kOwn:
                        // the slot (b0 + u) % kOwn is known at compile time.
                        // The sums are kept as they are; the level scale, the
                        // attention weight and the off-map test are applied
                        // once per owned sample after the loop.
                        if (li == lp / kOwn) {
#pragma unroll
                            for (int k = 0; k < kOwn; ++k) {
                                if ((b0 + u) % kOwn == k) {
                                    keep_w[k] = sw;
                                    keep_x[k] = sx;
                                    keep_y[k] = sy;
                                }
                            }
                        }
                    } else if (li == b0 + u) {
                        const int l = lp / P;                // uniform across the wave
                        own_w = off ? 0.0f : sw;
                        if constexpr (REF == 0) {
                            own_x = off ? 0.0f : sx * (static_cast<float>(pb.lv.W[l]) * fr.z);
                            own_y = off ? 0.0f : sy * (static_cast<float>(pb.lv.H[l]) * fr.z);
                        } else {
                            // d loc / d offset: 1 / (W, H) for 2-d reference
                            // points, ref_wh * 0.5 / P for 4-d ones
                            own_x = off ? 0.0f : sx * fr.z;
                            own_y = off ? 0.0f : sy * fr.z;
                            own_l = l;
                        }
                    }
                }
            }
            if (kOwn == 1 && li < kC) {
                const int64_t s = G * LP + c0 + li;
                if constexpr (REF == 0) {
                    store_scalar<ST>(grad_w, s, own_w);
                } else {
                    sv[lg * LP + c0 + li] = own_w;       // the softmax backward below
                    if constexpr (REF == 4) {
                        const int64_t ri = (static_cast<int64_t>(t.b) * pb.Q + t.q0 + lg) * L +
                                           own_l;
                        const float2 wh = load_pair<ST>(ref, 2 * ri + 1);
                        const float k = 0.5f / static_cast<float>(P);
                        own_x = own_x * static_cast<float>(pb.lv.W[own_l]) * (wh.x * k);
                        own_y = own_y * static_cast<float>(pb.lv.H[own_l]) * (wh.y * k);
                    }
                }
                store_pair<ST>(grad_loc, s, own_x, own_y);
            }
        }
        if constexpr (kOwn > 1) {
            // the owned samples kOwn * li + k: gradients scaled by (W_l, H_l)
            // times the attention weight, exactly zero for a sample off the
            // map (cell kNoCell: all four corners off the map; the plain form
            // has no key padding)
#pragma unroll
            for (int k = 0; k < kOwn; ++k) {
                const int lp = kOwn * li + k;
                const float4 fr = *reinterpret_cast<const float4*>(rec + lp * 8 + 4);    // lx ly w cell
                const int4 lv = s_lv[lp / P];
                const bool off = __float_as_uint(fr.w) == kNoCell;
                keep_w[k] = off ? 0.0f : keep_w[k];
                keep_x[k] = off ? 0.0f : keep_x[k] * (static_cast<float>(lv.y) * fr.z);
                keep_y[k] = off ? 0.0f : keep_y[k] * (static_cast<float>(lv.x) * fr.z);
            }
            constexpr int SE = Elem<ST>::bytes;
            const int64_t s0 = G * LP + kOwn * li;
            float xy[2 * kOwn];
#pragma unroll
            for (int k = 0; k < kOwn; ++k) {
                xy[2 * k] = keep_x[k];
                xy[2 * k + 1] = keep_y[k];
            }
            char* gl = static_cast<char*>(grad_loc) + s0 * 2 * SE;
            store_raw<16>(gl, narrow<ST, 16>(xy));
            if constexpr (2 * kOwn * SE == 32) store_raw<16>(gl + 16, narrow<ST, 16>(xy + 16 / SE));
            store_raw<kOwn * SE>(static_cast<char*>(grad_w) + s0 * SE, narrow<ST, kOwn * SE>(keep_w));
        }
    }
    if constexpr (REF != 0) {
        // softmax backward: with w the group's weights and g = dL/dw,
        // dL/dlogit_i = w_i * (g_i - sum_k w_k g_k)
        __syncthreads();
        for (int i = threadIdx.x; i < t.gcount * LP; i += blockDim.x) {
            const int g = i / LP;
            const uint32_t* r = srec + g * gstride + 6;          // the weights, 8 words apart
            const float* gg = sv + g * LP;
            float dot = 0.0f;
            for (int k = 0; k < LP; ++k) dot += __uint_as_float(r[8 * k]) * gg[k];
            const float wi = __uint_as_float(r[8 * (i - g * LP)]);
            store_scalar<ST>(grad_w, (t.G0 + static_cast<int64_t>(g) * pb.M) * LP + (i - g * LP), wi * (sv[i] - dot));
        }
    }
    if constexpr (!BINNED) {
        __syncthreads();
        pre_reduce_scatter<DT, VECB, LPR>(srec, gstride, LP, t.gcount, pre_g, pre_start, pre_end, pre_id,
                                          gacc + (static_cast<int64_t>(t.b) * pb.K * pb.M + t.m) * pb.D, pb);
    }
    if constexpr (BINNED) {
        __syncthreads();
        for (int i = threadIdx.x; i < pb.nseg; i += blockDim.x) {
            if (lhist[i] != 0) lbase[i] = atomicAdd(&cursor[static_cast<int64_t>(t.pl) * pb.nseg + i], lhist[i]);
            lhist[i] = 0;                            // reused as the record cursor
        }
        __syncthreads();
        // records, from the prologue's cell and weights in LDS, at base + a
        // slot taken from the segment's cursor
        const int64_t plane_end = (static_cast<int64_t>(t.pl) + 1) * 4 * pb.Q * LP;
        // Samples are walked point-major: consecutive lanes take consecutive
        // queries at one (level, point), whose records mostly fall in one
        // segment and take consecutive slots there.  A sample's (at most
        // four) records are formed first, then their slots are taken
        // together and the records stored.
        // (i < gcount * L * P <= kMaxWgSamples)
        const UDiv by_gcount = udiv_by(t.gcount);
        for (int i = threadIdx.x; i < t.gcount * LP; i += blockDim.x) {
            const int lp = udiv(i, by_gcount);
            const int g = i - lp * t.gcount, l = lp / P;
            const uint32_t* r = srec + g * gstride + lp * 8;
            const float4 fr = *reinterpret_cast<const float4*>(r + 4);    // lx ly w cell
            const uint32_t cell = __float_as_uint(fr.w);
            if (cell == kNoCell) continue;
            // the corner weights of rows y0 (w00, w01) and y0 + 1 (w10, w11)
            const float lx = fabsf(fr.x), ly = fabsf(fr.y);
            const float hx = 1.0f - lx, hy = 1.0f - ly;
            const float wy0 = fr.z * hy, wy1 = fr.z * ly;
            float w00 = wy0 * hx, w01 = wy0 * lx, w10 = wy1 * hx, w11 = wy1 * lx;
            // bit r: the record of image row y0 + r (the prologue marked the
            // rows whose record an earlier point of the level makes)
            const uint32_t rows = 3u & ~((__float_as_uint(fr.x) >> 31) | ((__float_as_uint(fr.y) >> 31) << 1));
            if (kMergeRecords<REF, L_CT, P_CT> && pb.merge_records != 0) {
                if (rows == 0u) continue;
                // record merging: this point's records carry the weights of
                // the later points' rows that they share (in point order)
                // (branch-free: a point that shares nothing adds zeros)
                const int p = lp % 4;
                const uint32_t* rl = r - p * 8;          // the level's point 0
                float4 fq[4];
#pragma unroll
                for (int q = 1; q < 4; ++q) fq[q] = *reinterpret_cast<const float4*>(rl + q * 8 + 4);
#pragma unroll
                for (int q = 1; q < 4; ++q) {
                    // point q's rows this one has (later points only)
                    const uint32_t sq = q > p ? shared_rows(__float_as_uint(fq[q].w), cell) : 0u;
                    const float qlx = fabsf(fq[q].x), qly = fabsf(fq[q].y);
                    const float qhx = 1.0f - qlx, qhy = 1.0f - qly;
                    const float qwy0 = fq[q].z * qhy, qwy1 = fq[q].z * qly;
                    // same cell: both rows; q's row y0 is this one's row
                    // y0 + 1 (sq 1); q's row y0 + 1 is this one's row y0 (sq 2)
                    const float a0 = sq == 3u ? qwy0 : (sq == 2u ? qwy1 : 0.0f);
                    const float a1 = sq == 3u ? qwy1 : (sq == 1u ? qwy0 : 0.0f);
                    w00 += a0 * qhx;
                    w01 += a0 * qlx;
                    w10 += a1 * qhx;
                    w11 += a1 * qlx;
                }
            }
            const int4 lv = s_lv[l];
            const int H = lv.x, W = lv.y, shift = lv.w & 0xff, segbase = lv.w >> 8;
            const int x0 = static_cast<int>(cell & 0xffffu) - 1, y0 = static_cast<int>(cell >> 16) - 1;
            const bool lin = x0 >= 0, rin = x0 + 1 < W;
            const uint32_t qk = static_cast<uint32_t>(t.q0 + g) << 8;
            const int kmask = (1 << shift) - 1;
            int seg[4], pos[4];
            uint3 rec[4];
            bool valid[4];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int yc = y0 + rr;
                const bool rowok = yc >= 0 && yc < H;
                const int kl = yc * W + x0, kr = kl + 1;
                const bool split = lin && rin && (kl >> shift) != (kr >> shift);
                const float cl = rr ? w10 : w00, cr = rr ? w11 : w01;
                const int k1 = lin ? kl : kr;
                valid[2 * rr] = rowok && ((rows >> rr) & 1u) != 0u;
                seg[2 * rr] = segbase + (k1 >> shift);
                rec[2 * rr] = make_uint3(qk | static_cast<uint32_t>(k1 & kmask), __float_as_uint(lin ? cl : cr),
                                         __float_as_uint(lin && rin && !split ? cr : 0.0f));
                valid[2 * rr + 1] = valid[2 * rr] && split;
                seg[2 * rr + 1] = segbase + (kr >> shift);
                rec[2 * rr + 1] = make_uint3(qk | static_cast<uint32_t>(kr & kmask), __float_as_uint(cr), 0u);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (valid[k]) pos[k] = lbase[seg[k]] + atomicAdd(&lhist[seg[k]], 1);
            // (positions past the plane's record region arise only from
            // counts of other locations, see msda_bin_scan_kernel: dropped)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (valid[k] && pos[k] < plane_end) recs[pos[k]] = rec[k];
        }
        // workgroup 0 also lays the planes' units out in one dense order for
        // the accumulation: units before each plane, and their total
        if (blockIdx.x == 0 && threadIdx.x < 64) {
            const int lane = threadIdx.x;
            int run = 0;
            for (int c0 = 0; c0 < pb.nplanes; c0 += 64) {
                const int v = c0 + lane < pb.nplanes ? nunits[c0 + lane] : 0;
                int inc = v;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int up = __shfl_up(inc, o, 64);
                    if (lane >= o) inc += up;
                }
                if (c0 + lane < pb.nplanes) nunits[2 * pb.nplanes + c0 + lane] = run + inc - v;
                run += __shfl(inc, 63, 64);
            }
            if (lane == 0) nunits[3 * pb.nplanes] = run;
        }
        // this plane's multi-unit segments, spread over the plane's workgroups
        const int nm = nunits[pb.nplanes + t.pl];
        const int nqc = (pb.Q + gpb - 1) / gpb;
        for (int e = t.q0 / gpb; e < nm; e += nqc)
            zero_segment(pb, gacc, multi[static_cast<int64_t>(t.pl) * pb.nseg + e], threadIdx.x, blockDim.x);
    }
}

// ---------------------------------------------------------------------------
// 4. accumulate
// ---------------------------------------------------------------------------
// Grid: nplanes * plane_units (the bound), acc_block(LPR, UNIT) lanes;
// workgroups past the total unit count exit, and the others take the units
// of all planes in plane order (nunits[2 nplanes + p]: units before plane p,
// written by the gradient kernel; nunits[3 nplanes]: all units), remapped so
// that each XCD gets a contiguous run.  LDS: the segment tile (keys * D
// floats), the unit's records sorted by key (UNIT weight pairs and keys,
// padded), 2 * kMaxSegKeys int32.
// UNIT / 32 workers of LPR lanes (at most 1024 lanes, at most one lane per
// record slot): the number of slice boundaries per record, and so the LDS
// compare-and-swap work, stays the same for every row width.  UNIT is
// kUnitRecords, or kSparseUnitRecords for sparse problems, whose units are
// many and short: smaller units and tiles let more of them run per CU.
constexpr int acc_block(int lpr, int unit) {
    return (unit / 32) * lpr < 1024 ? ((unit / 32) * lpr < unit ? (unit / 32) * lpr : unit)
                                    : (1024 < unit ? 1024 : unit);
}
// Sorted record i: key at word i + 4 * (i / 32), weight pair at pair slot
// i + 2 * (i / 32).  Workers start 8-aligned batches about 32 records apart
// and read them with 16-byte vector reads; the padding keeps those reads
// aligned and puts the eight workers of a wave in different LDS banks.
constexpr int sorted_key_slots(int unit) { return unit + unit / 8 + 8; }
constexpr int sorted_pair_slots(int unit) { return unit + unit / 16 + 8; }
__device__ __forceinline__ int key_slot(int i) { return i + 4 * (i >> 5); }
__device__ __forceinline__ int pair_slot(int i) { return i + 2 * (i >> 5); }

template <int DTK, int VECB, int LPR, int UNIT>
__global__ void __launch_bounds__(acc_block(LPR, UNIT), value_dt(DTK) == kF32 ? 6 : 5)
msda_accumulate_kernel(const void* __restrict__ gout, const uint3* __restrict__ recs,
                       const int32_t* __restrict__ nunits, const int4* __restrict__ units,
                       const uint8_t* __restrict__ kmask, float* __restrict__ gacc, void* __restrict__ gfinal,
                       Problem pb, int plane_units) {
    constexpr int DT = value_dt(DTK);                 // the accumulation touches no per-sample tensor
    constexpr int E = Elem<DT>::bytes;
    constexpr int VEC = VECB / E;
    constexpr int kAccBlock = acc_block(LPR, UNIT);
    constexpr int kAccPerLane = UNIT / kAccBlock;
    static_assert(kAccPerLane * kAccBlock == UNIT, "the unit's records split evenly over the lanes");
    constexpr int NW = kAccBlock / LPR;              // workers
    // consecutive units (neighbouring segments of one plane) run on one XCD,
    // so the plane's grad_output rows they gather stay in that XCD's L2
    // (clamped to the grid and to [0, np): the words come from the gradient
    // kernel's workgroup 0, and the host launches this kernel only after a
    // gradient kernel with at least one workgroup)
    const int np = pb.nplanes, lane = threadIdx.x & 63;
    // (the first 64 planes' unit prefixes load together with the total, not
    // after it: one memory round trip fewer before the unit is known)
    const int v0 = lane < np ? nunits[2 * np + lane] : 0x7fffffff;
    const int total = min(nunits[3 * np], static_cast<int>(gridDim.x));
    if (static_cast<int>(blockIdx.x) >= total) return;
    // workgroups 0 .. total-1 cover the units; each XCD gets a contiguous run
    const int r = static_cast<int>(xcd_tile(blockIdx.x, total));
    // the unit's plane: the number of planes whose first unit is <= r, less
    // one, counted 64 planes per load with a ballot
    int lo = -1;
    for (int c0 = 0; c0 < np; c0 += 64) {
        const int v = c0 == 0 ? v0 : (c0 + lane < np ? nunits[2 * np + c0 + lane] : 0x7fffffff);
        const int k = __popcll(__ballot(v <= r));
        lo += k;
        if (k < 64) break;
    }
    lo = min(max(lo, 0), np - 1);
    const int ui = min(max(r - nunits[2 * np + lo], 0), plane_units - 1);
    const int4 unit = units[static_cast<int64_t>(lo) * plane_units + ui];
    const int pl = unit.x / pb.nseg, seg = unit.x - pl * pb.nseg;
    const int b = pl / pb.M, m = pl - b * pb.M;
    const int lvl = level_of_segment(pb, seg);
    const int shift = pb.seg_shift[lvl];
    const int k0 = (seg - pb.seg_base[lvl]) << shift;
    const int nk = min(1 << shift, pb.lv.H[lvl] * pb.lv.W[lvl] - k0);
    const int n = unit.z - unit.y;
    const int D = pb.D;

    extern __shared__ float smem[];
    float* tile = smem;                                                  // nk * D
    float2* sw = reinterpret_cast<float2*>(smem + (1 << shift) * D);     // sorted weights
    uint32_t* skey = reinterpret_cast<uint32_t*>(sw + sorted_pair_slots(UNIT)); // sorted keys
    int32_t* hist = reinterpret_cast<int32_t*>(skey + sorted_key_slots(UNIT));
    int32_t* cur = hist + kMaxSegKeys;

    // (16-byte stores: nk * D is a multiple of 8)
    for (int i = threadIdx.x; i < nk * D / 4; i += kAccBlock)
        reinterpret_cast<float4*>(tile)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int i = threadIdx.x; i < kMaxSegKeys; i += kAccBlock) hist[i] = 0;
    __syncthreads();
    // counting sort by the key byte: records are read once, coalesced, and
    // held in registers until their sorted slot is known
    uint3 rec[kAccPerLane];
    if (n > 0) {
        // all loads in flight together (positions past n re-read the last record)
#pragma unroll
        for (int j = 0; j < kAccPerLane; ++j) {
            // non-temporal: the records are read once and would otherwise
            // evict the grad_output rows the fold gathers from L2 (encoder
            // accumulation 104 -> 96 us)
            const uint3* p = recs + unit.y + min(static_cast<int>(threadIdx.x) + j * kAccBlock, n - 1);
            rec[j] = make_uint3(__builtin_nontemporal_load(&p->x), __builtin_nontemporal_load(&p->y),
                                __builtin_nontemporal_load(&p->z));
        }
#pragma unroll
        for (int j = 0; j < kAccPerLane; ++j)
            if (static_cast<int>(threadIdx.x) + j * kAccBlock < n) atomicAdd(&hist[rec[j].x & 0xffu], 1);
    }
    __syncthreads();
    if (threadIdx.x < 64) {                          // exclusive scan of 256 bins, one wave
        const int lane = threadIdx.x;
        int v[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { v[j] = hist[4 * lane + j]; sum += v[j]; }
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int up = __shfl_up(incl, o, 64);
            if (lane >= o) incl += up;
        }
        int run = incl - sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) { cur[4 * lane + j] = run; run += v[j]; }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kAccPerLane; ++j) {
        const int i = threadIdx.x + j * kAccBlock;
        if (i < n) {
            const int pos = atomicAdd(&cur[rec[j].x & 0xffu], 1);
            skey[key_slot(pos)] = rec[j].x;
            sw[pair_slot(pos)] = make_float2(__uint_as_float(rec[j].y), __uint_as_float(rec[j].z));
        }
    }
    // pad to whole 8-record batches: the largest key, zero weights and a
    // query index one past the last, whose grad_output reads fall outside the
    // buffer and return zeros
    const int n8 = (n + 7) & ~7;
    if (static_cast<int>(threadIdx.x) < n8 - n) {
        skey[key_slot(n + threadIdx.x)] = (static_cast<uint32_t>(pb.Q) << 8) | 0xffu;
        sw[pair_slot(n + threadIdx.x)] = make_float2(0.0f, 0.0f);
    }
    __syncthreads();

    // Workers (LPR lanes each) walk equal 8-aligned slices of the sorted records,
    // accumulating rows key and key + 1 in registers while the key holds.
    // Rows kf..kf+1 and kl..kl+1 of a slice may also receive contributions
    // from neighbouring workers and are merged with LDS adds; every other row
    // is this worker's alone and is stored.  Records are taken kBatch at a
    // time: the worker loads their grad_output rows together, then folds
    // them in key order.
    constexpr int kBatch = 8;
    const int w = threadIdx.x / LPR, li = threadIdx.x % LPR;
    const bool active = li < pb.lpr_active;
    static_assert(kBatch == 8, "batches are read as two 16-byte key vectors");
    const int nb = n8 / kBatch;                      // whole 8-record batches
    const int r0 = kBatch * static_cast<int>(static_cast<int64_t>(nb) * w / NW);
    const int r1 = kBatch * static_cast<int>(static_cast<int64_t>(nb) * (w + 1) / NW);
    if (r0 < r1) {
        const int kf = static_cast<int>(skey[key_slot(r0)] & 0xffu);
        const int kl = static_cast<int>(skey[key_slot(r1 - 1)] & 0xffu);
        const int64_t gplane = static_cast<int64_t>(b) * pb.Q * pb.M + m;      // group (b, 0, m)
        const __amdgpu_buffer_rsrc_t gr = make_rsrc(
            static_cast<const char*>(gout) + gplane * D * E,
            static_cast<uint32_t>((static_cast<int64_t>(pb.Q) * pb.M - m) * D * E));
        const uint32_t qstride = static_cast<uint32_t>(pb.M * D * E);
        // lanes past the row read zeros through an out-of-range offset
        const uint32_t lane_b = active ? static_cast<uint32_t>(li * VECB) : kOffMap;
        auto flush = [&](int row, const float* acc) {
            if (!active || row >= nk) return;
            float* dst = tile + row * D + li * VEC;
            if (row > kf + 1 && row < kl) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) dst[i] = acc[i];
            } else {
                lds_add_f32xN<VEC>(dst, acc);
            }
        };
        float accA[VEC], accB[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) accA[i] = accB[i] = 0.0f;
        int key = kf;
        for (int base = r0; base < r1; base += kBatch) {
            int bkey[kBatch];
            float2 bw[kBatch];
            Raw<VECB> graw[kBatch];
            // the batch's 8 keys and weight pairs: 2 + 4 vector reads
            const uint4 ka = *reinterpret_cast<const uint4*>(skey + key_slot(base));
            const uint4 kb = *reinterpret_cast<const uint4*>(skey + key_slot(base) + 4);
            const float4 wa = *reinterpret_cast<const float4*>(sw + pair_slot(base));
            const float4 wb = *reinterpret_cast<const float4*>(sw + pair_slot(base) + 2);
            const float4 wc = *reinterpret_cast<const float4*>(sw + pair_slot(base) + 4);
            const float4 wd = *reinterpret_cast<const float4*>(sw + pair_slot(base) + 6);
            const uint32_t rr[kBatch] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
            const float2 ww[kBatch] = {make_float2(wa.x, wa.y), make_float2(wa.z, wa.w), make_float2(wb.x, wb.y),
                                       make_float2(wb.z, wb.w), make_float2(wc.x, wc.y), make_float2(wc.z, wc.w),
                                       make_float2(wd.x, wd.y), make_float2(wd.z, wd.w)};
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                bkey[j] = static_cast<int>(rr[j] & 0xffu);
                bw[j] = ww[j];
                // (24-bit products are exact here: query indices are below
                // 2^24, the row pitch M * D * E below 2^14, and the byte
                // offset below 2^31)
                graw[j] = buffer_load<VECB>(gr, __umul24(rr[j] >> 8, qstride) + lane_b);
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int rk = bkey[j];
                if (rk != key) {
                    flush(key, accA);
                    if (rk == key + 1) {
#pragma unroll
                        for (int i = 0; i < VEC; ++i) accA[i] = accB[i];
                    } else {
                        flush(key + 1, accB);
#pragma unroll
                        for (int i = 0; i < VEC; ++i) accA[i] = 0.0f;
                    }
#pragma unroll
                    for (int i = 0; i < VEC; ++i) accB[i] = 0.0f;
                    key = rk;
                }
                float gv[VEC];
                widen<DT, VECB>(graw[j], gv);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    accA[i] += bw[j].x * gv[i];
                    accB[i] += bw[j].y * gv[i];
                }
            }
        }
        flush(key, accA);
        flush(key + 1, accB);
    }
    __syncthreads();

    // Write the segment's rows: row k is key start + k0 + k of plane (b, m).
    // A segment split over several units adds with float atomics, lane i on
    // element i of a row (the lane-contiguous pattern), into the float32
    // buffer gacc.  Otherwise the rows are complete: one 16-byte
    // non-temporal store per lane (grad_value is not read again here),
    // float32 into gacc, or for 16-bit dtypes 8 elements rounded once
    // straight into grad_value (gfinal).
    const int64_t row0 = (static_cast<int64_t>(b) * pb.K + pb.lv.start[lvl] + k0) * pb.M + m;
    // rows of padded keys (the module zero-fills them, so their gradient is
    // zero) are written as zeros
    const uint8_t* km = kmask ? kmask + static_cast<int64_t>(b) * pb.K + pb.lv.start[lvl] + k0 : nullptr;
    // (divisions of i < nk * D <= 2^16 by D or less)
    const UDiv by_d = udiv_by(D);
    if (km != nullptr) {                             // uniform: a kernel argument
        for (int i = threadIdx.x; i < nk * D; i += kAccBlock)
            if (km[udiv(i, by_d)] != 0) tile[i] = 0.0f;
        __syncthreads();
    }
    if (unit.w) {
        for (int i = threadIdx.x; i < nk * D; i += kAccBlock) {
            const int k = udiv(i, by_d), d = i - k * D;
            if (km == nullptr || km[k] == 0)
                atomic_add_f32(gacc + (row0 + static_cast<int64_t>(k) * pb.M) * D + d, tile[i]);
        }
    } else if constexpr (DT == kF32) {
        const int q4 = D / 4;
        const UDiv by_q4 = udiv_by(q4);
        for (int i = threadIdx.x; i < nk * q4; i += kAccBlock) {
            const int k = udiv(i, by_q4), c4 = i - k * q4;
            const float4 v = *reinterpret_cast<const float4*>(tile + k * D + 4 * c4);
            float4* dst = reinterpret_cast<float4*>(gacc + (row0 + static_cast<int64_t>(k) * pb.M) * D + 4 * c4);
            __builtin_nontemporal_store(v.x, &dst->x); __builtin_nontemporal_store(v.y, &dst->y);
            __builtin_nontemporal_store(v.z, &dst->z); __builtin_nontemporal_store(v.w, &dst->w);
        }
    } else {
        const int q8 = D / 8;
        const UDiv by_q8 = udiv_by(q8);
        for (int i = threadIdx.x; i < nk * q8; i += kAccBlock) {
            const int k = udiv(i, by_q8), c8 = i - k * q8;
            const float* src = tile + k * D + 8 * c8;
            const Raw<16> r = narrow<DT, 16>(src);
            const int64_t e = (row0 + static_cast<int64_t>(k) * pb.M) * D + 8 * c8;
            uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(gfinal) + e * 2);
            __builtin_nontemporal_store(r.w[0], &dst->x); __builtin_nontemporal_store(r.w[1], &dst->y);
            __builtin_nontemporal_store(r.w[2], &dst->z); __builtin_nontemporal_store(r.w[3], &dst->w);
        }
    }
}

}  // namespace msda
