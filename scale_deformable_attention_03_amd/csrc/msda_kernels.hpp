// MSDeformAttn core kernels for gfx950: forward gather, backward
// gather + scatter, and the two small helpers of the backward (zero fill,
// float32 -> fp16/bf16 conversion).
//
// What is computed: "Deformable DETR walkthrough" (zhangshiyu.com/post/59697),
// section 2.2.4, ms_deform_attn_core_pytorch -- per level bilinear
// grid_sample (zeros padding, align_corners=False) at the L*P locations of a
// (batch, query, head), weighted by the attention weights and summed.
//
// Mapping.  A workgroup of 256 lanes owns GPB = 256/LPR consecutive groups
// (b, q, m).  It first stages the groups' locations and weights (contiguous
// in memory) into LDS as float32, then each group's LPR lanes walk the L*P
// samples: level geometry comes from launch arguments (scalar registers),
// the four corner rows are coalesced VECB-byte-per-lane reads, and the
// weighted corners are accumulated in float32 registers.  The path is a
// gather; there is no dense contraction, so no MFMA.
#pragma once

#include "msda_device.hpp"

namespace msda {

constexpr int kBlock = 256;

// LDS footprint of one workgroup (float words): per group, 2*LP location
// words (+2 padding so neighbouring groups start on different banks) and LP
// weight words (+1).
__host__ __device__ constexpr int lds_words(int gpb, int lp) {
    return gpb * (2 * lp + 2) + gpb * (lp + 1);
}

// Stage the locations and weights of groups [g0, g0 + gcount) into LDS.
template <int DT>
__device__ __forceinline__ void stage_tile(const void* __restrict__ loc, const void* __restrict__ attw,
                                           float* sloc, float* sw, int64_t g0, int gcount, int LP) {
    const int two_lp = 2 * LP;
    const int nloc = gcount * two_lp;
    const int64_t loc0 = g0 * two_lp;
    for (int i = threadIdx.x; i < nloc; i += kBlock) {
        int g = i / two_lp;
        sloc[g * (two_lp + 2) + (i - g * two_lp)] = load_scalar<DT>(loc, loc0 + i);
    }
    const int nw = gcount * LP;
    const int64_t w0 = g0 * LP;
    for (int i = threadIdx.x; i < nw; i += kBlock) {
        int g = i / LP;
        sw[g * (LP + 1) + (i - g * LP)] = load_scalar<DT>(attw, w0 + i);
    }
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <int DT, int VECB, int LPR, int L_CT, int P_CT>
__global__ void __launch_bounds__(kBlock)
msda_forward_kernel(const void* __restrict__ value, const void* __restrict__ loc,
                    const void* __restrict__ attw, void* __restrict__ out, Problem pb) {
    constexpr int E = Elem<DT>::bytes;
    constexpr int VEC = VECB / E;
    constexpr int GPB = kBlock / LPR;
    const int L = L_CT ? L_CT : pb.L;
    const int P = P_CT ? P_CT : pb.P;
    const int LP = L * P;

    extern __shared__ float smem[];
    float* sloc = smem;
    float* sw = smem + GPB * (2 * LP + 2);

    const int64_t g0 = xcd_tile(blockIdx.x, gridDim.x) * GPB;
    const int gcount = static_cast<int>(min(static_cast<int64_t>(GPB), pb.ngroups - g0));
    stage_tile<DT>(loc, attw, sloc, sw, g0, gcount, LP);
    __syncthreads();

    const int lg = threadIdx.x / LPR, li = threadIdx.x % LPR;
    if (lg >= gcount || li >= pb.lpr_active) return;

    const int64_t G = g0 + lg;
    const int m = static_cast<int>(G % pb.M);
    const int b = static_cast<int>((G / pb.M) / pb.Q);
    const int pitch = pb.M * pb.D;
    const char* vb = static_cast<const char*>(value) +
                     (static_cast<int64_t>(b) * pb.K * pitch + static_cast<int64_t>(m) * pb.D +
                      li * VEC) * E;
    const float* my_loc = sloc + lg * (2 * LP + 2);
    const float* my_w = sw + lg * (LP + 1);

    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;

#pragma unroll
    for (int l = 0; l < L; ++l) {
        const int H = pb.lv.H[l], W = pb.lv.W[l], start = pb.lv.start[l];
        const float Hf = static_cast<float>(H), Wf = static_cast<float>(W);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int lp = l * P + p;
            float x, y;
            if (!pixel_coords(my_loc[2 * lp], my_loc[2 * lp + 1], Wf, Hf, x, y)) continue;
            const Cell c = make_cell(x, y, W, H, start, pitch);
            const float aw = my_w[lp];
            const float wy0 = aw * c.hy, wy1 = aw * c.ly;
            const float w00 = wy0 * c.hx, w01 = wy0 * c.lx, w10 = wy1 * c.hx, w11 = wy1 * c.lx;
            float v[VEC];
            if (c.v00) {
                widen<DT, VECB>(load_raw<VECB>(vb + static_cast<int64_t>(c.off00) * E), v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] += w00 * v[i];
            }
            if (c.v01) {
                widen<DT, VECB>(load_raw<VECB>(vb + static_cast<int64_t>(c.off00 + c.dx) * E), v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] += w01 * v[i];
            }
            if (c.v10) {
                widen<DT, VECB>(load_raw<VECB>(vb + static_cast<int64_t>(c.off00 + c.dy) * E), v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] += w10 * v[i];
            }
            if (c.v11) {
                widen<DT, VECB>(load_raw<VECB>(vb + static_cast<int64_t>(c.off00 + c.dy + c.dx) * E), v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] += w11 * v[i];
            }
        }
    }
    char* ob = static_cast<char*>(out) + (G * pb.D + li * VEC) * E;
    store_raw<VECB>(ob, narrow<DT, VECB>(acc));
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------
__device__ __forceinline__ void atomic_add_f32(float* p, float v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int VEC>
__device__ __forceinline__ void scatter_row(float* p, float cw, const float* g) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) atomic_add_f32(p + i, cw * g[i]);
}

// gacc: float32 grad_value accumulator [bs, K, M, D], zeroed beforehand.
template <int DT, int VECB, int LPR, int L_CT, int P_CT>
__global__ void __launch_bounds__(kBlock)
msda_backward_kernel(const void* __restrict__ value, const void* __restrict__ loc,
                     const void* __restrict__ attw, const void* __restrict__ gout,
                     float* __restrict__ gacc, void* __restrict__ grad_loc,
                     void* __restrict__ grad_w, Problem pb) {
    constexpr int E = Elem<DT>::bytes;
    constexpr int VEC = VECB / E;
    constexpr int GPB = kBlock / LPR;
    const int L = L_CT ? L_CT : pb.L;
    const int P = P_CT ? P_CT : pb.P;
    const int LP = L * P;

    extern __shared__ float smem[];
    float* sloc = smem;
    float* sw = smem + GPB * (2 * LP + 2);

    const int64_t g0 = xcd_tile(blockIdx.x, gridDim.x) * GPB;
    const int gcount = static_cast<int>(min(static_cast<int64_t>(GPB), pb.ngroups - g0));
    stage_tile<DT>(loc, attw, sloc, sw, g0, gcount, LP);
    __syncthreads();

    const int lg = threadIdx.x / LPR, li = threadIdx.x % LPR;
    if (lg >= gcount) return;            // whole groups leave together
    const bool active = li < pb.lpr_active;

    const int64_t G = g0 + lg;
    const int m = static_cast<int>(G % pb.M);
    const int b = static_cast<int>((G / pb.M) / pb.Q);
    const int pitch = pb.M * pb.D;
    const int64_t vofs = static_cast<int64_t>(b) * pb.K * pitch + static_cast<int64_t>(m) * pb.D + li * VEC;
    const char* vb = static_cast<const char*>(value) + vofs * E;
    float* gb = gacc + vofs;
    const float* my_loc = sloc + lg * (2 * LP + 2);
    const float* my_w = sw + lg * (LP + 1);

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
            if (ok && active) {
                const Cell c = make_cell(x, y, W, H, start, pitch);
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
                const float wy0 = aw * c.hy, wy1 = aw * c.ly;
                if (c.v00) scatter_row<VEC>(gb + c.off00, wy0 * c.hx, g);
                if (c.v01) scatter_row<VEC>(gb + c.off00 + c.dx, wy0 * c.lx, g);
                if (c.v10) scatter_row<VEC>(gb + c.off00 + c.dy, wy1 * c.hx, g);
                if (c.v11) scatter_row<VEC>(gb + c.off00 + c.dy + c.dx, wy1 * c.lx, g);
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
}

// ---------------------------------------------------------------------------
// Helpers of the backward
// ---------------------------------------------------------------------------

// Zero n16 16-byte words (a fill kernel rather than a memset node, so the
// backward stays correct when a caller captures it in a HIP graph).
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

}  // namespace msda
