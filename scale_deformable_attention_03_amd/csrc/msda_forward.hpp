// MSDeformAttn core forward kernel for gfx950 (a gather).
//
// What is computed: "Deformable DETR walkthrough" (zhangshiyu.com/post/59697),
// section 2.2.4, ms_deform_attn_core_pytorch -- per level bilinear
// grid_sample (zeros padding, align_corners=False) at the L*P locations of a
// (batch, query, head), weighted by the attention weights and summed.
//
// Mapping.  A workgroup owns gpb consecutive queries of one (batch, head)
// plane; consecutive workgroups walk a plane's queries, and the XCD-aware
// block order gives each XCD contiguous runs of them, so a plane's value
// rows (K * D elements) stay in that XCD's L2.
//   prologue   one lane per sample (two or four per lane, with vector loads,
//              where kPrologueSamples allows): pixel coordinates, the cell's
//              four corner byte offsets within the plane (kOffMap for a
//              corner off the map) and the four corner weights times the
//              attention weight, into LDS (8 words per sample);
//   main loop  LPR lanes per query, VECB bytes of the D channels per lane:
//              per sample, two broadcast LDS reads, four raw-buffer loads
//              (off-map corners read as zeros) and 4*VEC FMAs into float32
//              registers; no branches.
// The path is a gather; there is no dense contraction, so no MFMA.
#pragma once

#include "msda_device.hpp"

namespace msda {

// Byte offsets of a sample's four corners within its (batch, head) plane of
// value (row pitch `pitch` bytes) and its bilinear cell.  Off-map samples get
// kOffMap offsets and zero fractions, with ok = false.
struct Corners {
    uint32_t o00, o01, o10, o11;
    float hx, lx, hy, ly;
    int x0, y0;
    bool ok;
};

__device__ __forceinline__ Corners sample_corners(float loc_x, float loc_y, int H, int W, int start,
                                                  uint32_t pitch) {
    Corners c;
    float x, y;
    c.ok = pixel_coords(loc_x, loc_y, static_cast<float>(W), static_cast<float>(H), x, y);
    if (!c.ok) {
        c.o00 = c.o01 = c.o10 = c.o11 = kOffMap;
        c.hx = c.lx = c.hy = c.ly = 0.0f;
        c.x0 = c.y0 = 0;
        return c;
    }
    const float fx = floorf(x), fy = floorf(y);
    c.x0 = static_cast<int>(fx);
    c.y0 = static_cast<int>(fy);
    c.lx = x - fx;
    c.ly = y - fy;
    c.hx = 1.0f - c.lx;
    c.hy = 1.0f - c.ly;
    const bool inx0 = c.x0 >= 0, inx1 = c.x0 + 1 < W, iny0 = c.y0 >= 0, iny1 = c.y0 + 1 < H;
    const int row = start + c.y0 * W + c.x0;          // may be negative; used only when in map
    c.o00 = (iny0 & inx0) ? static_cast<uint32_t>(row) * pitch : kOffMap;
    c.o01 = (iny0 & inx1) ? static_cast<uint32_t>(row + 1) * pitch : kOffMap;
    c.o10 = (iny1 & inx0) ? static_cast<uint32_t>(row + W) * pitch : kOffMap;
    c.o11 = (iny1 & inx1) ? static_cast<uint32_t>(row + W + 1) * pitch : kOffMap;
    return c;
}

// Key padding: the module fills the value rows of padded keys with zeros
// before the core ("Deformable DETR walkthrough", section 2.2.4,
// MSDeformAttn.forward), so a corner on a padded key reads as zero, exactly
// like a corner off the map.  km: the batch's num_keys mask bytes (nonzero =
// padded), or null for no padding.
__device__ __forceinline__ void mask_corners(Corners& c, const uint8_t* km, int start, int W) {
    if (km == nullptr || !c.ok) return;
    const int row = start + c.y0 * W + c.x0;          // in the map whenever o00 is
    if (c.o00 != kOffMap && km[row] != 0) c.o00 = kOffMap;
    if (c.o01 != kOffMap && km[row + 1] != 0) c.o01 = kOffMap;
    if (c.o10 != kOffMap && km[row + W] != 0) c.o10 = kOffMap;
    if (c.o11 != kOffMap && km[row + W + 1] != 0) c.o11 = kOffMap;
}

// Plane-local workgroup: queries q0 .. q0 + gcount - 1 of plane (b, m).
struct PlaneTile {
    int b, m, q0, gcount, pl;
    int64_t G0;        // flattened group (b, q0, m)
};

__device__ __forceinline__ PlaneTile plane_tile(const Problem& pb, int gpb) {
    PlaneTile t;
    const int nqc = (pb.Q + gpb - 1) / gpb;
    const int tile = static_cast<int>(xcd_tile(blockIdx.x, gridDim.x));
    t.pl = tile / nqc;
    const int qc = tile - t.pl * nqc;
    t.b = t.pl / pb.M;
    t.m = t.pl - t.b * pb.M;
    t.q0 = qc * gpb;
    t.gcount = min(gpb, pb.Q - t.q0);
    t.G0 = (static_cast<int64_t>(t.b) * pb.Q + t.q0) * pb.M + t.m;
    return t;
}

// Raw-buffer view of the value rows of plane (b, m): from element
// (b, 0, m, 0) to the end of batch b.
template <int E>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t value_plane(const void* value, const Problem& pb, int b, int m) {
    const int64_t batch = static_cast<int64_t>(pb.K) * pb.M * pb.D;
    const char* base = static_cast<const char*>(value) + (b * batch + static_cast<int64_t>(m) * pb.D) * E;
    return make_rsrc(base, static_cast<uint32_t>((batch - static_cast<int64_t>(m) * pb.D) * E));
}

// Grid: nplanes * ceil(Q / gpb) workgroups of gpb * LPR lanes.
// LDS: gpb * (8 * L * P + 4) words, plus 2 * gpb * L * P when REF != 0, plus
// nseg words when CNT.
// REF = 0: loc and attw are the sampling locations and attention weights;
// REF = 2 or 4: they are the sampling offsets and attention logits, and ref
// holds the reference points (see sample_location).  kmask: [bs, K] key
// padding bytes or null (see mask_corners).
// CNT (plain form only): the workgroup also counts its samples' backward
// records per segment (the binned backward's counting pass, done here from
// the cells the prologue computes anyway) and adds its counts into row
// (query tile mod nchunks) of its plane's histogram rows `counts` (one row
// per plane as launched), which the caller zeroed.
template <int DTK, int VECB, int LPR, int L_CT, int P_CT, int REF, bool CNT>
__global__ void __launch_bounds__(kBlock)
msda_forward_kernel(const void* __restrict__ value, const void* __restrict__ loc,
                    const void* __restrict__ attw, const void* __restrict__ ref,
                    const uint8_t* __restrict__ kmask, void* __restrict__ out, Problem pb, int gpb,
                    int32_t* __restrict__ counts, int nchunks) {
    static_assert(!CNT || REF == 0, "counting is built for the plain form");
    constexpr int DT = value_dt(DTK), ST = sample_dt(DTK);
    constexpr int E = Elem<DT>::bytes;
    constexpr int VEC = VECB / E;
    const int L = L_CT ? L_CT : pb.L;
    const int P = P_CT ? P_CT : pb.P;
    const int LP = L * P;
    const int gstride = 8 * LP + 4;

    extern __shared__ uint32_t sm[];
    const PlaneTile t = plane_tile(pb, gpb);
    const uint32_t pitch = static_cast<uint32_t>(pb.M * pb.D * E);
    __shared__ int4 s_lv[kMaxLevels];
    stage_levels(pb, s_lv);
    // fused prologue: the workgroup's logits and their exponentials
    float* sv = reinterpret_cast<float*>(sm + gpb * gstride);
    float* se = sv + gpb * LP;
    int32_t* lhist = reinterpret_cast<int32_t*>(sm + gpb * gstride);   // CNT: records per segment
    if constexpr (REF != 0) load_logits<ST>(attw, t.G0, pb.M, t.gcount, LP, sv);
    if constexpr (CNT)
        for (int i = threadIdx.x; i < pb.nseg; i += blockDim.x) lhist[i] = 0;
    __syncthreads();
    if constexpr (REF != 0) {
        exp_logits(t.gcount, LP, sv, se);
        __syncthreads();
    }

    // prologue: sample i = g * LP + lp of the workgroup, its corners c (from
    // its location) and (REF == 0) its attention weight w_in -> LDS record;
    // CNT: its records on the image rows in `rows` (bit r for row y0 + r: all,
    // or those record merging leaves it) are counted
    auto corners_of = [&](int lp, float2 xy) {
        const int4 lv = s_lv[lp / P];
        Corners c = sample_corners(xy.x, xy.y, lv.x, lv.y, lv.z, pitch);
        mask_corners(c, kmask ? kmask + static_cast<int64_t>(t.b) * pb.K : nullptr, lv.z, lv.y);
        return c;
    };
    auto stage = [&](int i, int g, int lp, const Corners& c, float w_in, uint32_t rows) {
        const int4 lv = s_lv[lp / P];
        float aw;
        if constexpr (REF == 0) aw = c.ok ? w_in : 0.0f;
        else aw = c.ok ? se[i] / group_total(se + g * LP, LP) : 0.0f;
        const float wy0 = aw * c.hy, wy1 = aw * c.ly;
        uint32_t* r = sm + g * gstride + lp * 8;
        *reinterpret_cast<uint4*>(r) = make_uint4(c.o00, c.o01, c.o10, c.o11);
        *reinterpret_cast<float4*>(r + 4) = make_float4(wy0 * c.hx, wy0 * c.lx, wy1 * c.hx, wy1 * c.lx);
        if constexpr (CNT) {
            if (c.ok && rows != 0u)
                for_each_record(
                    c.x0, c.y0, lv.y, lv.x, lv.w & 0xff, lv.w >> 8,
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
            // each sample's record goes to LDS as soon as its corners are
            // known; only its packed cell stays for the counting below (so
            // the counting forward's prologue holds S cells, not S corner sets)
            uint32_t cell[S], rows[S];
#pragma unroll
            for (int k = 0; k < S; ++k) {
                const Corners c = corners_of(lp + k, make_float2(xy[2 * k], xy[2 * k + 1]));
                stage(i + k, g, lp + k, c, wv[k], 0u);
                cell[k] = c.ok ? pack_cell(c.x0, c.y0) : kNoCell;
                rows[k] = 3u;
            }
            if constexpr (CNT) {
                if constexpr (kMergeRecords<REF, L_CT, P_CT>) {
                    // (the lane pair holding a level's four points is active
                    // together: t.gcount * LP and the loop stride are multiples
                    // of four)
                    if (pb.merge_records) record_rows<S>(cell, lp % P, rows);
                }
#pragma unroll
                for (int k = 0; k < S; ++k) {
                    if (cell[k] == kNoCell) continue;
                    const int4 lv = s_lv[(lp + k) / P];
                    for_each_record(
                        static_cast<int>(cell[k] & 0xffffu) - 1, static_cast<int>(cell[k] >> 16) - 1, lv.y, lv.x,
                        lv.w & 0xff, lv.w >> 8, [&](int seg, int, int, int) { atomicAdd(&lhist[seg], 1); }, rows[k]);
                }
            }
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
    if constexpr (CNT) {
        int32_t* row = counts + (static_cast<int64_t>(t.pl) * nchunks + (t.q0 / gpb) % nchunks) * pb.nseg;
        for (int i = threadIdx.x; i < pb.nseg; i += blockDim.x) {
            const int v = lhist[i];
            if (v != 0) atomicAdd(row + i, v);
        }
    }

    const int lg = threadIdx.x / LPR, li = threadIdx.x % LPR;
    if (lg >= t.gcount || li >= pb.lpr_active) return;
    const __amdgpu_buffer_rsrc_t vr = value_plane<E>(value, pb, t.b, t.m);
    const uint32_t lane_b = static_cast<uint32_t>(li * VECB);
    const uint32_t* rec = sm + lg * gstride;

    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
    // samples whose loads fly together; bf16 widens each element with its own
    // shift or mask, so fewer of its rows are held at once
    constexpr int kSBMax = DT == kBF16 ? 2 : 4;
    constexpr int kSB = L_CT && P_CT && (L_CT * P_CT) % kSBMax == 0 ? kSBMax : 1;
    // 16-bit values widen to twice the registers: at most two batches unrolled
    constexpr int kUnroll = E == 4 ? 4 : (DT == kF16 ? 2 : 1);
#pragma unroll kUnroll
    for (int lp0 = 0; lp0 < LP; lp0 += kSB) {
        float4 w[kSB];
        Raw<VECB> raw[kSB][4];
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            const uint4 o = *reinterpret_cast<const uint4*>(rec + (lp0 + u) * 8);
            w[u] = *reinterpret_cast<const float4*>(rec + (lp0 + u) * 8 + 4);
            raw[u][0] = buffer_load<VECB>(vr, o.x + lane_b);
            raw[u][1] = buffer_load<VECB>(vr, o.y + lane_b);
            raw[u][2] = buffer_load<VECB>(vr, o.z + lane_b);
            raw[u][3] = buffer_load<VECB>(vr, o.w + lane_b);
        }
        // a batch of several samples: its loads all go out before the first
        // fold (measured: the large-batch bf16 forward 301 -> 293 us, the
        // fp16 decoder's 12.2 -> 9.5 us; the one-sample batches of the generic
        // kernel keep the compiler's own interleaving, which is faster there)
        if constexpr (kSB > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            if constexpr (DT == kBF16) {
                // one corner row at a time: each widened element feeds its FMA
                // at once, so few widened values are live together
                const float wc[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float v[VEC];
                    widen<DT, VECB>(raw[u][c], v);
#pragma unroll
                    for (int i = 0; i < VEC; ++i) acc[i] += wc[c] * v[i];
                }
            } else {
                float v0[VEC], v1[VEC], v2[VEC], v3[VEC];
                widen<DT, VECB>(raw[u][0], v0);
                widen<DT, VECB>(raw[u][1], v1);
                widen<DT, VECB>(raw[u][2], v2);
                widen<DT, VECB>(raw[u][3], v3);
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    acc[i] += w[u].x * v0[i] + w[u].y * v1[i] + w[u].z * v2[i] + w[u].w * v3[i];
            }
        }
    }
    const int64_t G = t.G0 + static_cast<int64_t>(lg) * pb.M;
    store_raw<VECB>(static_cast<char*>(out) + (G * pb.D + li * VEC) * E, narrow<DT, VECB>(acc));
}

}  // namespace msda
