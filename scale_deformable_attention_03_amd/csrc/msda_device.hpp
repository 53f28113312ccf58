// Device-side building blocks shared by the MSDeformAttn kernels (gfx950).
//
// Data layout (see include/msda.h): value [bs, K, M, D]; a (batch, query,
// head) triple is a "group" G = (b*Q + q)*M + m.  Its locations are the
// L*P*2 contiguous elements at G*L*P*2, its weights the L*P elements at
// G*L*P, its output (and grad_output) the D elements at G*D.  A group is
// processed by LPR consecutive lanes; each active lane owns VEC consecutive
// channels (VECB bytes), so a bilinear corner is one coalesced row read of
// D*e bytes spread over the group's lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msda_types.hpp"

namespace msda {

// ---- per-level table in LDS ------------------------------------------------

// Per-sample code indexes the level table with a per-lane level, which from
// kernel arguments would be a vector memory load per sample; a workgroup
// copies the table into LDS once instead.  Row l: (H, W, start, seg), seg =
// segment shift | first segment << 8.
__device__ __forceinline__ void stage_levels(const Problem& pb, int4* lt) {
    for (int l = threadIdx.x; l < pb.L; l += blockDim.x)
        lt[l] = make_int4(pb.lv.H[l], pb.lv.W[l], pb.lv.start[l], pb.seg_shift[l] | (pb.seg_base[l] << 8));
}

// ---- scalar conversions --------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
    _Float16 h = __builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16));
    return static_cast<float>(h);
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    _Float16 h = static_cast<_Float16>(f);   // v_cvt_f16_f32: round to nearest even
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

template <int DT>
__device__ __forceinline__ float load_scalar(const void* base, int64_t i) {
    if constexpr (DT == kF32) {
        return static_cast<const float*>(base)[i];
    } else if constexpr (DT == kF16) {
        return f16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
    } else {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
    }
}

template <int DT>
__device__ __forceinline__ void store_scalar(void* base, int64_t i, float v) {
    if constexpr (DT == kF32) {
        static_cast<float*>(base)[i] = v;
    } else if constexpr (DT == kF16) {
        static_cast<uint16_t*>(base)[i] = static_cast<uint16_t>(f32_to_f16_bits(v));
    } else {
        static_cast<uint16_t*>(base)[i] = static_cast<uint16_t>(f32_to_bf16_bits(v));
    }
}

// Elements 2i and 2i + 1 (a location's x and y) in one load / one store.
template <int DT>
__device__ __forceinline__ float2 load_pair(const void* base, int64_t i) {
    if constexpr (DT == kF32) {
        return static_cast<const float2*>(base)[i];
    } else {
        const uint32_t w = static_cast<const uint32_t*>(base)[i];
        if constexpr (DT == kF16) return make_float2(f16_bits_to_f32(w & 0xffffu), f16_bits_to_f32(w >> 16));
        else return make_float2(bf16_bits_to_f32(w & 0xffffu), bf16_bits_to_f32(w >> 16));
    }
}

template <int DT>
__device__ __forceinline__ void store_pair(void* base, int64_t i, float a, float b) {
    if constexpr (DT == kF32) {
        static_cast<float2*>(base)[i] = make_float2(a, b);
    } else if constexpr (DT == kF16) {
        static_cast<uint32_t*>(base)[i] = f32_to_f16_bits(a) | (f32_to_f16_bits(b) << 16);
    } else {
        static_cast<uint32_t*>(base)[i] = f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
    }
}

// a.lo * b.lo + a.hi * b.hi + c for two packed 16-bit pairs (fp16 or bf16),
// float32 result: the products of 16-bit values are exact in float32.
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (DT == kF16) {
        typedef _Float16 __attribute__((ext_vector_type(2))) h2;
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
    } else {
        typedef __bf16 __attribute__((ext_vector_type(2))) b2;
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
    }
}

// ---- vector row slices -------------------------------------------------------

// VECB raw bytes of a row, held in 32-bit words.
template <int VECB> struct Raw { uint32_t w[VECB / 4]; };

// load_raw / store_raw move the data each kernel streams once (sampling
// locations and weights, a query's grad_output row, outputs and gradients)
// with non-temporal loads and stores, so that they do not push out of L2 the
// value and grad_output rows that the gathers reuse (measured on the
// large-batch bf16 encoder step: 1.233 -> 1.200 ms).  The gathers themselves
// use buffer loads (below).

template <int VECB>
__device__ __forceinline__ Raw<VECB> load_raw(const void* p) {
    Raw<VECB> r;
    if constexpr (VECB == 16) {
        const uint4* q = static_cast<const uint4*>(p);
        r.w[0] = __builtin_nontemporal_load(&q->x); r.w[1] = __builtin_nontemporal_load(&q->y);
        r.w[2] = __builtin_nontemporal_load(&q->z); r.w[3] = __builtin_nontemporal_load(&q->w);
    } else if constexpr (VECB == 8) {
        const uint2* q = static_cast<const uint2*>(p);
        r.w[0] = __builtin_nontemporal_load(&q->x); r.w[1] = __builtin_nontemporal_load(&q->y);
    } else {
        r.w[0] = __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
    }
    return r;
}

template <int VECB>
__device__ __forceinline__ void store_raw(void* p, const Raw<VECB>& r) {
    if constexpr (VECB == 16) {
        uint4* q = static_cast<uint4*>(p);
        __builtin_nontemporal_store(r.w[0], &q->x); __builtin_nontemporal_store(r.w[1], &q->y);
        __builtin_nontemporal_store(r.w[2], &q->z); __builtin_nontemporal_store(r.w[3], &q->w);
    } else if constexpr (VECB == 8) {
        uint2* q = static_cast<uint2*>(p);
        __builtin_nontemporal_store(r.w[0], &q->x); __builtin_nontemporal_store(r.w[1], &q->y);
    } else {
        __builtin_nontemporal_store(r.w[0], static_cast<uint32_t*>(p));
    }
}

// Widen VECB bytes of dtype DT into VEC floats (element 0 in the low bits).
template <int DT, int VECB>
__device__ __forceinline__ void widen(const Raw<VECB>& r, float* out) {
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < VECB / 4; ++i) out[i] = __uint_as_float(r.w[i]);
    } else if constexpr (DT == kF16) {
#pragma unroll
        for (int i = 0; i < VECB / 4; ++i) {
            out[2 * i] = f16_bits_to_f32(r.w[i] & 0xffffu);
            out[2 * i + 1] = f16_bits_to_f32(r.w[i] >> 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < VECB / 4; ++i) {
            out[2 * i] = __uint_as_float(r.w[i] << 16);
            out[2 * i + 1] = __uint_as_float(r.w[i] & 0xffff0000u);
        }
    }
}

// Round VEC floats to dtype DT (nearest even) and pack into VECB bytes.
template <int DT, int VECB>
__device__ __forceinline__ Raw<VECB> narrow(const float* in) {
    Raw<VECB> r;
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < VECB / 4; ++i) r.w[i] = __float_as_uint(in[i]);
    } else if constexpr (DT == kF16) {
#pragma unroll
        for (int i = 0; i < VECB / 4; ++i)
            r.w[i] = f32_to_f16_bits(in[2 * i]) | (f32_to_f16_bits(in[2 * i + 1]) << 16);
    } else {
#pragma unroll
        for (int i = 0; i < VECB / 4; ++i)
            r.w[i] = f32_to_bf16_bits(in[2 * i]) | (f32_to_bf16_bits(in[2 * i + 1]) << 16);
    }
    return r;
}

// ---- buffer loads ------------------------------------------------------------

// Raw buffer descriptor over `bytes` bytes from `base` (gfx9 word 3).  A load
// whose offset lies at or beyond `bytes` returns zeros, which is how corners
// off the map are read: their offset is set to kOffMap.
constexpr uint32_t kOffMap = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

template <int VECB>
__device__ __forceinline__ Raw<VECB> buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Raw<VECB> out;
    if constexpr (VECB == 16) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0);
        out.w[0] = v[0]; out.w[1] = v[1]; out.w[2] = v[2]; out.w[3] = v[3];
    } else if constexpr (VECB == 8) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, 0);
        out.w[0] = v[0]; out.w[1] = v[1];
    } else {
        out.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0);
    }
    return out;
}

// ---- sampling geometry ---------------------------------------------------------

// Pixel coordinates of a normalised location under align_corners=False:
// x = loc_x*W - 0.5, y = loc_y*H - 0.5, each product and difference rounded
// to float32 on its own (contraction off: a fused multiply-add would move
// exact pixel centres such as 0.005*100 - 0.5 off the integer grid).
// Returns whether the sample touches the map: -1 < x < W and -1 < y < H
// (NaN fails).
__device__ __forceinline__ bool pixel_coords(float loc_x, float loc_y, float Wf, float Hf,
                                             float& x, float& y) {
#pragma clang fp contract(off)
    x = loc_x * Wf;
    x = x - 0.5f;
    y = loc_y * Hf;
    y = y - 0.5f;
    return (x > -1.0f) & (x < Wf) & (y > -1.0f) & (y < Hf);
}

// ---- sampling locations and weights (plain or fused prologue) --------------
//
// REF selects what the kernels are given.  REF = 0: sampling locations
// [bs,Q,M,L,P,2] and attention weights [bs,Q,M,L,P].  REF = 2 or 4: the step
// before the core in "Deformable DETR walkthrough" section 2.2.4
// (MSDeformAttn.forward): reference points [bs,Q,L,REF], sampling offsets
// laid out like the locations and attention logits laid out like the
// weights.  The location is ref + offset / (W, H) for 2-d reference points
// and ref_xy + offset / P * ref_wh * 0.5 for 4-d ones, each operation rounded
// to float32 in that order; the weights are the softmax of the L*P logits of
// one (batch, query, head).

// Sample si's location; ri = (b * Q + q) * L + l indexes its reference point.
template <int DT, int REF>
__device__ __forceinline__ float2 sample_location(const void* loc_or_off, const void* ref, int64_t si,
                                                  int64_t ri, float Wf, float Hf, float Pf) {
#pragma clang fp contract(off)
    const float2 a = load_pair<DT>(loc_or_off, si);
    if constexpr (REF == 0) {
        return a;
    } else if constexpr (REF == 2) {
        const float2 r = load_pair<DT>(ref, ri);
        const float ox = a.x / Wf, oy = a.y / Hf;
        return make_float2(r.x + ox, r.y + oy);
    } else {
        const float2 rxy = load_pair<DT>(ref, 2 * ri), rwh = load_pair<DT>(ref, 2 * ri + 1);
        float tx = a.x / Pf, ty = a.y / Pf;
        tx = tx * rwh.x;
        ty = ty * rwh.y;
        tx = tx * 0.5f;
        ty = ty * 0.5f;
        return make_float2(rxy.x + tx, rxy.y + ty);
    }
}

// Samples per lane in the prologues: S = 16 / (2 * sample bytes) (2 for
// float32 locations and weights, 4 for 16-bit ones), so that one 16-byte
// load holds a lane's S locations and one 8-byte load its S weights.  Taken
// for the plain form (not the fused one) when L * P is fixed and a multiple
// of S, so a lane's samples never straddle two groups and its loads stay
// aligned; 1 (one sample per lane, scalar loads) otherwise.
template <int ST, int REF, int L_CT, int P_CT>
constexpr int kPrologueSamples =
    REF == 0 && L_CT != 0 && P_CT != 0 && (L_CT * P_CT) % (8 / Elem<ST>::bytes) == 0 ? 8 / Elem<ST>::bytes : 1;

// Softmax of each (batch, query, head)'s L*P logits, staged through LDS for
// the gcount groups G0, G0 + M, ... of a workgroup (sample i = g * LP + lp):
// load_logits fills sv; after a barrier exp_logits writes
// se[i] = exp(sv[i] - max of the group); after another barrier a sample's
// weight is se[i] / group_total(se + g * LP, LP).  Float32 throughout.
template <int DT>
__device__ __forceinline__ void load_logits(const void* logits, int64_t G0, int M, int gcount, int LP,
                                            float* sv) {
    for (int i = threadIdx.x; i < gcount * LP; i += blockDim.x) {
        const int g = i / LP, lp = i - g * LP;
        sv[i] = load_scalar<DT>(logits, (G0 + static_cast<int64_t>(g) * M) * LP + lp);
    }
}

__device__ __forceinline__ void exp_logits(int gcount, int LP, const float* sv, float* se) {
    for (int i = threadIdx.x; i < gcount * LP; i += blockDim.x) {
        const float* v = sv + (i / LP) * LP;
        float mx = v[0];
        for (int k = 1; k < LP; ++k) mx = fmaxf(mx, v[k]);
        se[i] = expf(sv[i] - mx);
    }
}

__device__ __forceinline__ float group_total(const float* a, int n) {
    float s = 0.0f;
    for (int k = 0; k < n; ++k) s += a[k];
    return s;
}

// Bilinear cell of a valid sample: the four corners' flat offsets (in
// elements, relative to the (batch, head) base), their in-map flags and
// bilinear weights (without the attention weight).
struct Cell {
    int32_t x0, y0;          // floor of the pixel coordinates
    int32_t off00;           // row (start + y0*W + x0) times the row pitch M*D
    int32_t dx, dy;          // offset steps to the x+1 and y+1 corners
    bool v00, v01, v10, v11;
    float lx, ly, hx, hy;
};

__device__ __forceinline__ Cell make_cell(float x, float y, int32_t W, int32_t H, int32_t start,
                                          int32_t pitch) {
    Cell c;
    float fx = floorf(x), fy = floorf(y);
    c.x0 = static_cast<int32_t>(fx);
    c.y0 = static_cast<int32_t>(fy);
    c.lx = x - fx;
    c.ly = y - fy;
    c.hx = 1.0f - c.lx;
    c.hy = 1.0f - c.ly;
    bool inx0 = c.x0 >= 0, inx1 = c.x0 + 1 < W, iny0 = c.y0 >= 0, iny1 = c.y0 + 1 < H;
    c.v00 = iny0 & inx0;
    c.v01 = iny0 & inx1;
    c.v10 = iny1 & inx0;
    c.v11 = iny1 & inx1;
    c.off00 = (start + c.y0 * W + c.x0) * pitch;
    c.dx = pitch;
    c.dy = W * pitch;
    return c;
}

// ---- division by a workgroup-uniform divisor --------------------------------------

// i / d for 0 <= i and 1 <= d with i * d < 2^32, as a multiply-high by
// ceil(2^32 / d) (d = 1 divides by taking i itself): two instructions in a
// loop instead of an integer division sequence.
struct UDiv {
    uint32_t m;
    int d;
};

__device__ __forceinline__ UDiv udiv_by(int d) {
    UDiv u;
    u.d = d;
    u.m = d > 1 ? 0xffffffffu / static_cast<uint32_t>(d) + 1u : 0u;
    return u;
}

__device__ __forceinline__ int udiv(int i, const UDiv& u) {
    return u.d > 1 ? static_cast<int>(__umulhi(static_cast<uint32_t>(i), u.m)) : i;
}

// ---- launch geometry -----------------------------------------------------------

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Remap so that each XCD walks one contiguous range of tiles: neighbouring
// query tiles (raster neighbours in an encoder) then share that XCD's L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t block, int64_t nblocks) {
    constexpr int64_t kXcd = 8;
    int64_t x = block % kXcd, i = block / kXcd;
    int64_t per = nblocks / kXcd, rem = nblocks % kXcd;
    return x * per + (x < rem ? x : rem) + i;
}

// Value of lane (pattern applied to this lane) through a DPP move: row_mirror
// (0x140) pairs lanes i and 15-i of a 16-lane row, row_half_mirror (0x141)
// lanes i and 7-i of an 8-lane half row, quad_perm 0x4E / 0xB1 lanes i^2 /
// i^1 of a quad.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the LPR lanes of a group (LPR a power of two, groups aligned):
// cross-row steps by lane permute, the rest by DPP within a row.  Every lane
// of the group ends with the total.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPR >= 64) v += __shfl_xor(v, 32, 64);
    if constexpr (LPR >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (LPR >= 16) v += dpp<0x140>(v);
    if constexpr (LPR >= 8) v += dpp<0x141>(v);
    if constexpr (LPR >= 4) {
        v += dpp<0x4E>(v);
        v += dpp<0xB1>(v);
    }
    return v;
}

// ---- records -----------------------------------------------------------------
// A record is one image row (y0 or y0 + 1) of one sample's bilinear cell,
// restricted to the row's in-map corners of one segment:
//   key   u32: query index << 8 | key of its first corner within the segment
//   w2    float2: weight of that key's corner and of the next key's corner
//         (0 when the row's second corner is off the map or in the next
//         segment), each w * (1-ly or ly) * (1-lx or lx)
constexpr uint32_t kNoCell = 0xffffffffu;  // packed cell of a sample off the map

// Corners of one row that a record covers.
enum RecMode : int { kBoth = 0, kLeftOnly = 1, kRightOnly = 2 };

// Packed cell (x0 + 1, y0 + 1) of an in-map sample (16-bit fields; never
// equal to kNoCell on levels of at most 65534 pixels a side).
__device__ __forceinline__ uint32_t pack_cell(int x0, int y0) {
    return static_cast<uint32_t>(x0 + 1) | (static_cast<uint32_t>(y0 + 1) << 16);
}

// Record merging.  The samples of one (batch, query, head, level) scale the
// same grad_output row, so records of two of them on the same image row with
// the same x-pair have the same keys.  In point order (a point's row y0
// before its row y0 + 1), the first such record is made, with the corner
// weights of the later ones added in that order, and the later ones are not.
// Built for the plain form at four points per level and fixed L * P, where
// the points of a query often lie within a pixel of each other on the coarse
// levels (about a quarter of the encoder's records); every count of records
// (count kernel, counting forward, the gradient kernel's own count) and the
// gradient kernel's records follow the same rule.
template <int REF, int L_CT, int P_CT>
constexpr bool kMergeRecords = REF == 0 && L_CT != 0 && P_CT == 4;

// Rows of the sample with packed cell cp (bit r: image row y0 + r) that a
// sample with packed cell cq also has (same x-pair, one or both rows in
// common); 0 when cq is kNoCell (its low field, 0xffff, is no in-map x0 + 1).
__device__ __forceinline__ uint32_t shared_rows(uint32_t cp, uint32_t cq) {
    if (((cp ^ cq) & 0xffffu) != 0u) return 0u;
    const int dy = static_cast<int>(cp >> 16) - static_cast<int>(cq >> 16);
    return dy == 0 ? 3u : (dy == 1 ? 1u : (dy == -1 ? 2u : 0u));
}

// rows[k]: the rows (bit r: image row y0 + r) for which the lane's sample k
// makes a record, i.e. no earlier point of its level has a record on that
// image row with the same x-pair.  The lane holds S consecutive samples of
// one level, points p0 .. p0 + S - 1 (p0 a multiple of S), with packed cells
// `cell` (kNoCell off the map: such a sample makes no records and its rows
// do not matter).  S == 2: the level's other two points are in lane ^ 1,
// which runs the same call (both lanes are active together).  S == 4: all
// four are here.
template <int S>
__device__ __forceinline__ void record_rows(const uint32_t (&cell)[S], int p0, uint32_t (&rows)[S]) {
    static_assert(S == 2 || S == 4, "a lane holds two or four points of a level");
    uint32_t c[4];
    if constexpr (S == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = cell[k];
        p0 = 0;
    } else {
        const uint32_t o0 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(cell[0]), 1, 64));
        const uint32_t o1 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(cell[1]), 1, 64));
        const bool hi = p0 != 0;                     // this lane holds points 2, 3
        c[0] = hi ? o0 : cell[0];
        c[1] = hi ? o1 : cell[1];
        c[2] = hi ? cell[0] : o0;
        c[3] = hi ? cell[1] : o1;
    }
#pragma unroll
    for (int k = 0; k < S; ++k) {
        uint32_t taken = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < p0 + k) taken |= shared_rows(cell[k], c[q]);
        rows[k] = 3u & ~taken;
    }
}

// Enumerate the records of a valid sample whose cell starts at (x0, y0) on
// a W x H level (-1 <= x0 < W, -1 <= y0 < H): for each of the rows y0,
// y0 + 1 that lie on the map (and are in `rows`, bit r for row y0 + r), the
// in-map corners of that row.  A pair whose
// two corners fall in different segments is split in two records.
// emit(segment, key within segment, row 0/1, mode).
template <typename Emit>
__device__ __forceinline__ void for_each_record(int x0, int y0, int W, int H, int shift, int segbase,
                                                Emit&& emit, uint32_t rows = 3u) {
    const int mask = (1 << shift) - 1;
    const bool lin = x0 >= 0, rin = x0 + 1 < W;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int yc = y0 + r;
        if (yc < 0 || yc >= H || ((rows >> r) & 1u) == 0u) continue;
        const int kl = yc * W + x0;    // left corner key (meaningful when lin)
        const int kr = kl + 1;         // right corner key
        if (lin && rin) {
            if ((kl >> shift) == (kr >> shift)) {
                emit(segbase + (kl >> shift), kl & mask, r, static_cast<int>(kBoth));
            } else {
                emit(segbase + (kl >> shift), kl & mask, r, static_cast<int>(kLeftOnly));
                emit(segbase + (kr >> shift), kr & mask, r, static_cast<int>(kRightOnly));
            }
        } else if (lin) {
            emit(segbase + (kl >> shift), kl & mask, r, static_cast<int>(kLeftOnly));
        } else {
            emit(segbase + (kr >> shift), kr & mask, r, static_cast<int>(kRightOnly));
        }
    }
}

}  // namespace msda
