// MSDeformAttn core forward kernel for gfx950 (a gather).
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
    stage_groups<DT>(loc, attw, sloc, sw, g0, 1, gcount, LP);
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

}  // namespace msda
