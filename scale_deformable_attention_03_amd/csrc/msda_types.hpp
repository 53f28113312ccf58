// Plain types and constants of the MSDeformAttn kernels, shared by the
// device code and the host planning code (msda_plan.hpp).  No HIP: the
// host planning code also builds with a plain C++ compiler (the sanitizer
// build of the tests).
#pragma once

#include <stdint.h>

namespace msda {

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Kernel dtype codes: kF32, kF16, kBF16 (every float tensor in that type),
// or mixed precision: kF16M / kBF16M keep value, output and their gradients
// in fp16 / bf16 and the per-sample tensors (locations or offsets, weights
// or logits, reference points, and their gradients) in float32.
constexpr int kF16M = 3, kBF16M = 4;
// type of the value-side tensors, and of the per-sample tensors
constexpr int value_dt(int code) { return code == kF16M ? kF16 : code == kBF16M ? kBF16 : code; }
constexpr int sample_dt(int code) { return code >= kF16M ? kF32 : code; }

template <int DT> struct Elem;
template <> struct Elem<kF32> { static constexpr int bytes = 4; };
template <> struct Elem<kF16> { static constexpr int bytes = 2; };
template <> struct Elem<kBF16> { static constexpr int bytes = 2; };

constexpr int kMaxLevels = 64;   // L*P <= 64 bounds L

// Level geometry as launch arguments: uniform across the grid, so the
// compiler keeps the entries it reads in scalar registers.
struct LevelTable {
    int32_t H[kMaxLevels];
    int32_t W[kMaxLevels];
    int32_t start[kMaxLevels];
};

struct Problem {
    int32_t bs, K, M, D, L, P, Q;
    int32_t lpr_active;      // lanes of a group that own channels
    int64_t ngroups;         // bs * Q * M
    LevelTable lv;
    // Key segments of the binned backward (see msda_backward.hpp): level l
    // is cut into segments of 2^seg_shift[l] keys, numbered from
    // seg_base[l] within a (batch, head) plane; seg_base[L] = nseg.
    int32_t nseg;
    int32_t nplanes;         // bs * M
    int32_t unit_records;    // records per accumulation unit (kUnitRecords or kSparseUnitRecords)
    int32_t merge_records;   // 1: the L4P4 kernels merge records (see kMergeRecords)
    int32_t seg_shift[kMaxLevels];
    int32_t seg_base[kMaxLevels + 1];
};

constexpr int kBlock = 256;   // lanes of a full workgroup

// Envelope and sizes of the binned backward (see msda_backward.hpp).
constexpr int kQueryBits = 24;         // queries per plane for the binned path
constexpr int kMaxSegKeys = 256;       // keys per segment (8-bit key field)
constexpr int kUnitRecords = 2048;     // records one accumulation unit sorts
constexpr int kSparseUnitRecords = 512; // the same for sparse problems (fewer than one record per key)
constexpr int kMaxSegments = 2048;     // segments per plane (LDS histograms)
constexpr int kMaxWgSamples = 1024;    // samples one gradient workgroup holds
constexpr int kMaxBinnedExtent = 65534; // H and W of a level on the binned path (16-bit cell fields)
constexpr int kCountBlock = 512;       // lanes of a counting workgroup
constexpr int kCountChunk = 4096;      // samples one counting workgroup bins (at least)
constexpr int kMaxCountChunks = 64;    // counting workgroups (histogram rows) per plane
// histogram rows per plane that a counting forward adds into (its
// workgroups add with integer atomics, so one row serves them all: the scan
// then sums one row instead of kMaxCountChunks)
constexpr int kForwardCountRows = 1;

constexpr int kCountScanSamples = 8192;  // samples of a plane counted and scanned by one workgroup
constexpr int kNarrowPerPlane = 8;     // workgroups per plane rounding multi-unit rows to 16 bits

}  // namespace msda
