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
// reductions over the embedding channels (wave shuffles), computed by the
// gradient kernel, which gathers the four corner rows exactly as the forward
// does.
//
// grad_value is a transposed gather: row (b, key, m) sums w * (bilinear
// weight) * grad_output[b, q, m] over every sample corner that lands on it.
// Scattering those D-wide contributions with float atomics costs one L2
// atomic per row per sample corner; measured on MI355X that path tops out
// near 340 G float updates/s, far below what the gather side runs at.  So the
// backward bins instead:
//
//   1. count     each (batch, head) plane's keys are cut into segments; every
//                in-map corner pair of a sample (the two corners of one image
//                row) becomes a 4-byte record; count records per segment
//                (LDS histograms, one global add per non-empty bin).
//   2. scan      exclusive prefix over the counts gives each segment a record
//                range and a cursor; segments are split into units of at most
//                kUnitRecords records.
//   3. gradient  the gather kernel (grad_w, grad_loc) also writes its records
//                at positions reserved per workgroup and segment.
//   4. accumulate  one workgroup per unit: counting-sort the unit's records by
//                key in LDS, let each worker (LPR lanes) walk a key-sorted slice
//                accumulating rows in registers, merge into an LDS tile, and
//                write every row of the segment once with plain stores (units
//                of a segment split in several use float atomics instead, into
//                rows the scan zeroed).
//
// Segment sizes per level are planned on the host from the expected records
// per key, so that most segments fit one unit.  Outside the envelope of the
// record format (see binned_ok on the host) the gradient kernel scatters
// grad_value with float atomics instead.
#pragma once

#include "msda_device.hpp"

namespace msda {

// ---- records -----------------------------------------------------------------
// A record is one image row of one sample's bilinear cell:
//   bits  0..20  sample index within its (batch, head) plane, q*L*P + l*P + p
//   bit   21     row: 0 = y0, 1 = y0 + 1
//   bits 22..23  corners: kBoth (key, key+1), kLeftOnly (key = x0 corner),
//                kRightOnly (key = x0+1 corner)
//   bits 24..31  key within its segment
constexpr int kRecSampleBits = 21;
constexpr uint32_t kRecSampleMask = (1u << kRecSampleBits) - 1u;
constexpr int kMaxSegKeys = 256;       // keys per segment (8-bit key field)
constexpr int kUnitRecords = 4096;     // records one accumulation unit sorts
constexpr int kMaxSegments = 2048;     // segments per plane (LDS histograms)
constexpr int kMaxWgRecords = 4096;    // records one gradient workgroup stages
constexpr int kCountChunk = 4096;      // samples one counting workgroup bins
constexpr int kScanThreads = 1024;
constexpr int kMultiList = 2048;

enum RecMode : uint32_t { kBoth = 0, kLeftOnly = 1, kRightOnly = 2 };

__device__ __forceinline__ uint32_t make_record(uint32_t s, uint32_t row, uint32_t mode, uint32_t key) {
    return s | (row << 21) | (mode << 22) | (key << 24);
}

// Enumerate the records of a valid sample whose cell starts at (x0, y0) on
// a W x H level (-1 <= x0 < W, -1 <= y0 < H): for each of the rows y0,
// y0 + 1 that lie on the map, the in-map corners of that row.  A pair whose
// two corners fall in different segments is split in two records.
template <typename Emit>
__device__ __forceinline__ void for_each_record(uint32_t s, int x0, int y0, int W, int H, int shift,
                                                int segbase, Emit&& emit) {
    const int mask = (1 << shift) - 1;
    const bool lin = x0 >= 0, rin = x0 + 1 < W;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int yc = y0 + r;
        if (yc < 0 || yc >= H) continue;
        const int kl = yc * W + x0;    // left corner key (meaningful when lin)
        const int kr = kl + 1;         // right corner key
        if (lin && rin) {
            if ((kl >> shift) == (kr >> shift)) {
                emit(make_record(s, r, kBoth, kl & mask), segbase + (kl >> shift));
            } else {
                emit(make_record(s, r, kLeftOnly, kl & mask), segbase + (kl >> shift));
                emit(make_record(s, r, kRightOnly, kr & mask), segbase + (kr >> shift));
            }
        } else if (lin) {
            emit(make_record(s, r, kLeftOnly, kl & mask), segbase + (kl >> shift));
        } else {
            emit(make_record(s, r, kRightOnly, kr & mask), segbase + (kr >> shift));
        }
    }
}

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
__global__ void __launch_bounds__(kBlock) msda_zero_kernel(uint4* __restrict__ p, int64_t n16) {
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

// ---------------------------------------------------------------------------
// 1. count
// ---------------------------------------------------------------------------
// Grid: nplanes * ceil(Q*L*P / kCountChunk) workgroups of kBlock lanes; one
// lane per sample.  LDS: nseg int32.
template <int DT, int L_CT, int P_CT>
__global__ void __launch_bounds__(kBlock)
msda_bin_count_kernel(const void* __restrict__ loc, int32_t* __restrict__ counts, Problem pb) {
    extern __shared__ int32_t hist[];
    const int L = L_CT ? L_CT : pb.L;
    const int P = P_CT ? P_CT : pb.P;
    const int LP = L * P;
    const int nsamp = pb.Q * LP;
    const int nchunks = (nsamp + kCountChunk - 1) / kCountChunk;
    const int pl = blockIdx.x / nchunks, chunk = blockIdx.x - pl * nchunks;
    const int b = pl / pb.M, m = pl - b * pb.M;

    for (int i = threadIdx.x; i < pb.nseg; i += kBlock) hist[i] = 0;
    __syncthreads();
    const int s_end = min((chunk + 1) * kCountChunk, nsamp);
    for (int s = chunk * kCountChunk + threadIdx.x; s < s_end; s += kBlock) {
        const int q = s / LP, lp = s - q * LP, l = lp / P;
        const int64_t i = ((static_cast<int64_t>(b) * pb.Q + q) * pb.M + m) * LP + lp;
        const int H = pb.lv.H[l], W = pb.lv.W[l];
        float x, y;
        if (!pixel_coords(load_scalar<DT>(loc, 2 * i), load_scalar<DT>(loc, 2 * i + 1),
                          static_cast<float>(W), static_cast<float>(H), x, y))
            continue;
        const int x0 = static_cast<int>(floorf(x)), y0 = static_cast<int>(floorf(y));
        for_each_record(static_cast<uint32_t>(s), x0, y0, W, H, pb.seg_shift[l], pb.seg_base[l],
                        [&](uint32_t, int seg) { atomicAdd(&hist[seg], 1); });
    }
    __syncthreads();
    for (int i = threadIdx.x; i < pb.nseg; i += kBlock)
        if (hist[i] != 0) atomicAdd(&counts[static_cast<int64_t>(pl) * pb.nseg + i], hist[i]);
}

// ---------------------------------------------------------------------------
// 2. scan
// ---------------------------------------------------------------------------

__device__ __forceinline__ int units_of(int count) {
    return count <= kUnitRecords ? 1 : (count + kUnitRecords - 1) / kUnitRecords;
}

// Zero the float32 rows of plane-global segment `gs`, lanes t, t+nt, ...
__device__ void zero_segment(const Problem& pb, float* gacc, int gs, int t, int nt) {
    const int pl = gs / pb.nseg, seg = gs - pl * pb.nseg;
    const int b = pl / pb.M, m = pl - b * pb.M;
    const int l = level_of_segment(pb, seg);
    const int k0 = (seg - pb.seg_base[l]) << pb.seg_shift[l];
    const int nk = min(1 << pb.seg_shift[l], pb.lv.H[l] * pb.lv.W[l] - k0);
    for (int i = t; i < nk * pb.D; i += nt) {
        const int k = i / pb.D, d = i - k * pb.D;
        const int64_t key = pb.lv.start[l] + k0 + k;
        gacc[((static_cast<int64_t>(b) * pb.K + key) * pb.M + m) * pb.D + d] = 0.0f;
    }
}

// One workgroup.  counts -> cursor (exclusive prefix), the unit list
// {segment, first record, end record, flush-with-atomics} and its length,
// and zeroed rows for segments split over several units.  With `accumulate`
// every unit adds into the caller's buffer, which is then left as it is.
__global__ void __launch_bounds__(kScanThreads)
msda_bin_scan_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ cursor,
                     int32_t* __restrict__ nunits, int4* __restrict__ units, float* __restrict__ gacc,
                     int accumulate, Problem pb) {
    __shared__ int32_t s_rec[kScanThreads], s_unit[kScanThreads];
    __shared__ int32_t s_multi[kMultiList];
    __shared__ int32_t s_nmulti;
    const int t = threadIdx.x;
    const int n = pb.nplanes * pb.nseg;
    const int per = (n + kScanThreads - 1) / kScanThreads;
    const int i0 = min(n, t * per), i1 = min(n, i0 + per);
    int rsum = 0, usum = 0;
    for (int i = i0; i < i1; ++i) {
        const int c = counts[i];
        rsum += c;
        usum += units_of(c);
    }
    s_rec[t] = rsum;
    s_unit[t] = usum;
    if (t == 0) s_nmulti = 0;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {     // inclusive scan
        const int a = t >= off ? s_rec[t - off] : 0;
        const int u = t >= off ? s_unit[t - off] : 0;
        __syncthreads();
        s_rec[t] += a;
        s_unit[t] += u;
        __syncthreads();
    }
    int rbase = s_rec[t] - rsum, ubase = s_unit[t] - usum;
    if (t == kScanThreads - 1) nunits[0] = s_unit[t];
    for (int i = i0; i < i1; ++i) {
        const int c = counts[i], u = units_of(c);
        cursor[i] = rbase;
        const int atomic_flush = (u > 1 || accumulate) ? 1 : 0;
        for (int j = 0; j < u; ++j)
            units[ubase + j] = make_int4(i, rbase + j * kUnitRecords, rbase + min(c, (j + 1) * kUnitRecords),
                                         atomic_flush);
        if (u > 1 && !accumulate) {
            const int k = atomicAdd(&s_nmulti, 1);
            if (k < kMultiList) s_multi[k] = i;
            else zero_segment(pb, gacc, i, 0, 1);
        }
        rbase += c;
        ubase += u;
    }
    __syncthreads();
    const int nm = min(s_nmulti, kMultiList);
    for (int k = 0; k < nm; ++k) zero_segment(pb, gacc, s_multi[k], t, kScanThreads);
}

// ---------------------------------------------------------------------------
// 3. gradient (gather): grad_w, grad_loc, and grad_value records or atomics
// ---------------------------------------------------------------------------
// Grid: nplanes * ceil(Q / gpb) workgroups of gpb * LPR lanes; workgroup
// (plane, chunk) owns queries chunk*gpb .. +gpb of that (batch, head).
// LDS: staged locations / weights (lds_words(gpb, LP) floats); when BINNED
// also nseg histogram + nseg bases (int32), per-group record counts and
// gpb*LP*4 record slots (two uint32 each).
template <int DT, int VECB, int LPR, int L_CT, int P_CT, bool BINNED>
__global__ void __launch_bounds__(kBlock)
msda_backward_kernel(const void* __restrict__ value, const void* __restrict__ loc,
                     const void* __restrict__ attw, const void* __restrict__ gout,
                     float* __restrict__ gacc, uint32_t* __restrict__ records,
                     int32_t* __restrict__ cursor, void* __restrict__ grad_loc,
                     void* __restrict__ grad_w, Problem pb, int gpb) {
    constexpr int E = Elem<DT>::bytes;
    constexpr int VEC = VECB / E;
    const int L = L_CT ? L_CT : pb.L;
    const int P = P_CT ? P_CT : pb.P;
    const int LP = L * P;

    extern __shared__ float smem[];
    float* sloc = smem;
    float* sw = smem + gpb * (2 * LP + 2);
    int32_t* lhist = reinterpret_cast<int32_t*>(smem + lds_words(gpb, LP));
    int32_t* lbase = lhist + pb.nseg;
    int32_t* gcnt = lbase + pb.nseg;
    uint32_t* lrec = reinterpret_cast<uint32_t*>(gcnt + gpb);
    uint32_t* lsr = lrec + gpb * LP * 4;

    const int nqc = (pb.Q + gpb - 1) / gpb;
    const int tile = static_cast<int>(xcd_tile(blockIdx.x, gridDim.x));
    const int pl = tile / nqc, qc = tile - pl * nqc;
    const int b = pl / pb.M, m = pl - b * pb.M;
    const int q0 = qc * gpb;
    const int gcount = min(gpb, pb.Q - q0);
    const int64_t G0 = (static_cast<int64_t>(b) * pb.Q + q0) * pb.M + m;

    if constexpr (BINNED) {
        for (int i = threadIdx.x; i < pb.nseg; i += blockDim.x) lhist[i] = 0;
    }
    stage_groups<DT>(loc, attw, sloc, sw, G0, pb.M, gcount, LP);
    __syncthreads();

    const int lg = threadIdx.x / LPR, li = threadIdx.x % LPR;
    if (lg < gcount) {
        const bool active = li < pb.lpr_active;
        const int64_t G = G0 + static_cast<int64_t>(lg) * pb.M;
        const int pitch = pb.M * pb.D;
        const int64_t vofs = static_cast<int64_t>(b) * pb.K * pitch + static_cast<int64_t>(m) * pb.D + li * VEC;
        const char* vb = static_cast<const char*>(value) + vofs * E;
        float* gb = gacc + vofs;
        const float* my_loc = sloc + lg * (2 * LP + 2);
        const float* my_w = sw + lg * (LP + 1);
        uint32_t* my_rec = lrec + lg * LP * 4;
        uint32_t* my_sr = lsr + lg * LP * 4;
        int nrec = 0;

        float g[VEC];
        if (active) {
            widen<DT, VECB>(load_raw<VECB>(static_cast<const char*>(gout) + (G * pb.D + li * VEC) * E), g);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) g[i] = 0.0f;
        }

#pragma unroll
        for (int l = 0; l < L; ++l) {
            const int H = pb.lv.H[l], W = pb.lv.W[l], start = pb.lv.start[l];
            const float Hf = static_cast<float>(H), Wf = static_cast<float>(W);
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int lp = l * P + p;
                float x, y;
                const bool ok = pixel_coords(my_loc[2 * lp], my_loc[2 * lp + 1], Wf, Hf, x, y);
                const float aw = my_w[lp];
                float gw = 0.0f, gx = 0.0f, gy = 0.0f;
                if (ok) {
                    const Cell c = make_cell(x, y, W, H, start, pitch);
                    if (active) {
                        float v00[VEC], v01[VEC], v10[VEC], v11[VEC];
#pragma unroll
                        for (int i = 0; i < VEC; ++i) v00[i] = v01[i] = v10[i] = v11[i] = 0.0f;
                        if (c.v00) widen<DT, VECB>(load_raw<VECB>(vb + static_cast<int64_t>(c.off00) * E), v00);
                        if (c.v01) widen<DT, VECB>(load_raw<VECB>(vb + static_cast<int64_t>(c.off00 + c.dx) * E), v01);
                        if (c.v10) widen<DT, VECB>(load_raw<VECB>(vb + static_cast<int64_t>(c.off00 + c.dy) * E), v10);
                        if (c.v11) widen<DT, VECB>(load_raw<VECB>(vb + static_cast<int64_t>(c.off00 + c.dy + c.dx) * E), v11);
#pragma unroll
                        for (int i = 0; i < VEC; ++i) {
                            const float top = c.hx * v00[i] + c.lx * v01[i];
                            const float bot = c.hx * v10[i] + c.lx * v11[i];
                            gw += g[i] * (c.hy * top + c.ly * bot);
                            gx += g[i] * (c.hy * (v01[i] - v00[i]) + c.ly * (v11[i] - v10[i]));
                            gy += g[i] * (bot - top);
                        }
                        if constexpr (!BINNED) {
                            const float wy0 = aw * c.hy, wy1 = aw * c.ly;
#pragma unroll
                            for (int i = 0; i < VEC; ++i) {
                                if (c.v00) atomic_add_f32(gb + c.off00 + i, wy0 * c.hx * g[i]);
                                if (c.v01) atomic_add_f32(gb + c.off00 + c.dx + i, wy0 * c.lx * g[i]);
                                if (c.v10) atomic_add_f32(gb + c.off00 + c.dy + i, wy1 * c.hx * g[i]);
                                if (c.v11) atomic_add_f32(gb + c.off00 + c.dy + c.dx + i, wy1 * c.lx * g[i]);
                            }
                        }
                    }
                    if constexpr (BINNED) {
                        if (li == 0) {
                            const uint32_t s = static_cast<uint32_t>((q0 + lg) * LP + lp);
                            for_each_record(s, c.x0, c.y0, W, H, pb.seg_shift[l], pb.seg_base[l],
                                            [&](uint32_t rec, int seg) {
                                                const int rank = atomicAdd(&lhist[seg], 1);
                                                my_rec[nrec] = rec;
                                                my_sr[nrec] = (static_cast<uint32_t>(seg) << 16) |
                                                              static_cast<uint32_t>(rank);
                                                ++nrec;
                                            });
                        }
                    }
                }
                gw = group_sum<LPR>(gw);
                gx = group_sum<LPR>(gx);
                gy = group_sum<LPR>(gy);
                if (li == 0) {
                    const int64_t s = G * LP + lp;
                    store_scalar<DT>(grad_w, s, gw);
                    store_scalar<DT>(grad_loc, 2 * s, ok ? Wf * aw * gx : 0.0f);
                    store_scalar<DT>(grad_loc, 2 * s + 1, ok ? Hf * aw * gy : 0.0f);
                }
            }
        }
        if constexpr (BINNED) {
            if (li == 0) gcnt[lg] = nrec;
        }
    }
    if constexpr (BINNED) {
        if (threadIdx.x / LPR >= gcount && threadIdx.x % LPR == 0 && threadIdx.x / LPR < gpb)
            gcnt[threadIdx.x / LPR] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < pb.nseg; i += blockDim.x)
            if (lhist[i] != 0) lbase[i] = atomicAdd(&cursor[static_cast<int64_t>(pl) * pb.nseg + i], lhist[i]);
        __syncthreads();
        const int slots = 4 * LP;
        for (int i = threadIdx.x; i < gpb * slots; i += blockDim.x) {
            const int grp = i / slots, j = i - grp * slots;
            if (j < gcnt[grp]) {
                const uint32_t sr = lsr[i];
                records[lbase[sr >> 16] + static_cast<int>(sr & 0xffffu)] = lrec[i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 4. accumulate
// ---------------------------------------------------------------------------
// Grid: an upper bound on the unit count, kBlock lanes; workgroups past
// nunits exit.  LDS: the segment tile (keys * D floats), kUnitRecords
// records (uint32) and their key order (uint16), 2 * kMaxSegKeys int32.
template <int DT, int VECB, int LPR, int L_CT, int P_CT>
__global__ void __launch_bounds__(kBlock)
msda_accumulate_kernel(const void* __restrict__ loc, const void* __restrict__ attw,
                       const void* __restrict__ gout, const uint32_t* __restrict__ records,
                       const int32_t* __restrict__ nunits, const int4* __restrict__ units,
                       float* __restrict__ gacc, Problem pb) {
    constexpr int E = Elem<DT>::bytes;
    constexpr int VEC = VECB / E;
    constexpr int NW = kBlock / LPR;                 // workers
    const int L = L_CT ? L_CT : pb.L;
    const int P = P_CT ? P_CT : pb.P;
    const int LP = L * P;
    if (static_cast<int>(blockIdx.x) >= nunits[0]) return;

    const int4 unit = units[blockIdx.x];
    const int pl = unit.x / pb.nseg, seg = unit.x - pl * pb.nseg;
    const int b = pl / pb.M, m = pl - b * pb.M;
    const int lvl = level_of_segment(pb, seg);
    const int shift = pb.seg_shift[lvl];
    const int k0 = (seg - pb.seg_base[lvl]) << shift;
    const int H = pb.lv.H[lvl], W = pb.lv.W[lvl];
    const int nk = min(1 << shift, H * W - k0);
    const int n = unit.z - unit.y;
    const int D = pb.D;

    extern __shared__ float smem[];
    float* tile = smem;                                            // nk * D
    uint32_t* recs = reinterpret_cast<uint32_t*>(smem + (1 << shift) * D);
    int32_t* hist = reinterpret_cast<int32_t*>(recs + kUnitRecords);
    int32_t* cur = hist + kMaxSegKeys;
    uint16_t* order = reinterpret_cast<uint16_t*>(cur + kMaxSegKeys);

    for (int i = threadIdx.x; i < nk * D; i += kBlock) tile[i] = 0.0f;
    for (int i = threadIdx.x; i < kMaxSegKeys; i += kBlock) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kBlock) {
        const uint32_t r = records[unit.y + i];
        recs[i] = r;
        atomicAdd(&hist[r >> 24], 1);
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
    for (int i = threadIdx.x; i < n; i += kBlock)
        order[atomicAdd(&cur[recs[i] >> 24], 1)] = static_cast<uint16_t>(i);
    __syncthreads();

    // Workers walk key-sorted slices; rows kf..kf+1 and kl..kl+1 of a slice
    // may also receive contributions from neighbouring workers and are merged
    // with LDS adds, every other row is this worker's alone.
    const int w = threadIdx.x / LPR, li = threadIdx.x % LPR;
    const bool active = li < pb.lpr_active;
    const int r0 = static_cast<int>(static_cast<int64_t>(n) * w / NW);
    const int r1 = static_cast<int>(static_cast<int64_t>(n) * (w + 1) / NW);
    if (r0 < r1) {
        const int kf = static_cast<int>(recs[order[r0]] >> 24), kl = static_cast<int>(recs[order[r1 - 1]] >> 24);
        const float Hf = static_cast<float>(H), Wf = static_cast<float>(W);
        auto flush = [&](int row, const float* acc) {
            if (!active || row >= nk) return;
            float* dst = tile + row * D + li * VEC;
            if (row > kf + 1 && row < kl) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) dst[i] = acc[i];
            } else {
#pragma unroll
                for (int i = 0; i < VEC; ++i) lds_add_f32(dst + i, acc[i]);
            }
        };
        float accA[VEC], accB[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) accA[i] = accB[i] = 0.0f;
        int key = -1;
        for (int r = r0; r < r1; ++r) {
            const uint32_t rec = recs[order[r]];
            const int rkey = static_cast<int>(rec >> 24);
            if (rkey != key) {
                if (key >= 0) {
                    flush(key, accA);
                    if (rkey == key + 1) {
#pragma unroll
                        for (int i = 0; i < VEC; ++i) accA[i] = accB[i];
                    } else {
                        flush(key + 1, accB);
#pragma unroll
                        for (int i = 0; i < VEC; ++i) accA[i] = 0.0f;
                    }
#pragma unroll
                    for (int i = 0; i < VEC; ++i) accB[i] = 0.0f;
                }
                key = rkey;
            }
            const int s = static_cast<int>(rec & kRecSampleMask);
            const int q = s / LP, lp = s - q * LP;
            const int64_t G = (static_cast<int64_t>(b) * pb.Q + q) * pb.M + m;
            const int64_t si = G * LP + lp;
            float x, y;
            pixel_coords(load_scalar<DT>(loc, 2 * si), load_scalar<DT>(loc, 2 * si + 1), Wf, Hf, x, y);
            const float fx = floorf(x), fy = floorf(y);
            const float lx = x - fx, ly = y - fy;
            const float aw = load_scalar<DT>(attw, si);
            const float wy = aw * (((rec >> 21) & 1u) ? ly : 1.0f - ly);
            const float cl = wy * (1.0f - lx), cr = wy * lx;
            const uint32_t mode = (rec >> 22) & 3u;
            const float ca = mode == kRightOnly ? cr : cl;
            const float cb = mode == kBoth ? cr : 0.0f;
            if (active) {
                float g[VEC];
                widen<DT, VECB>(load_raw<VECB>(static_cast<const char*>(gout) + (G * D + li * VEC) * E), g);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    accA[i] += ca * g[i];
                    accB[i] += cb * g[i];
                }
            }
        }
        flush(key, accA);
        flush(key + 1, accB);
    }
    __syncthreads();

    // Write the segment's rows: row k is key start + k0 + k of plane (b, m).
    const int atomic_flush = unit.w;
    const int q4 = D / 4;
    const int64_t row0 = (static_cast<int64_t>(b) * pb.K + pb.lv.start[lvl] + k0) * pb.M + m;
    for (int i = threadIdx.x; i < nk * q4; i += kBlock) {
        const int k = i / q4, c4 = i - k * q4;
        float* dst = gacc + (row0 + static_cast<int64_t>(k) * pb.M) * D + 4 * c4;
        const float* src = tile + k * D + 4 * c4;
        if (atomic_flush) {
            atomic_add_f32(dst + 0, src[0]);
            atomic_add_f32(dst + 1, src[1]);
            atomic_add_f32(dst + 2, src[2]);
            atomic_add_f32(dst + 3, src[3]);
        } else {
            *reinterpret_cast<float4*>(dst) = make_float4(src[0], src[1], src[2], src[3]);
        }
    }
}

}  // namespace msda
