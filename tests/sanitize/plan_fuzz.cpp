// Host planning code of libmsda (csrc/msda_plan.hpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer: fixed cases at the envelope's edges (the
// same descriptors as the C-ABI host tests) and a seeded fuzz, each checked
// against the invariants the kernels rely on.  Prints "plan_fuzz ok" and
// exits 0 when every check holds; the first failing check exits 1.
// Built and run by tests/test_sanitize_host.py (g++, no GPU).
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "msda_plan.hpp"

namespace {

int g_checks = 0;

#define EXPECT(cond, ...)                                                         \
    do {                                                                          \
        ++g_checks;                                                               \
        if (!(cond)) {                                                            \
            fprintf(stderr, "plan_fuzz: check failed at line %d: %s\n  ", __LINE__, #cond); \
            fprintf(stderr, __VA_ARGS__);                                         \
            fprintf(stderr, "\n");                                                \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

struct Desc {
    int bs = 2, M = 8, D = 32, P = 4, Q = 300, dtype = 0;
    std::vector<std::pair<int64_t, int64_t>> shapes{{100, 134}, {50, 67}, {25, 34}, {13, 17}};
    int64_t K = -1;                  // -1: the sum of H*W
    std::vector<int64_t> starts;     // empty: the exclusive prefix sum
    std::vector<int64_t> flat;       // storage of the host arrays

    msda_problem_t make() {
        flat.clear();
        for (auto& s : shapes) {
            flat.push_back(s.first);
            flat.push_back(s.second);
        }
        int64_t sum = 0;
        std::vector<int64_t> st;
        for (auto& s : shapes) {
            st.push_back(sum);
            sum += s.first * s.second;
        }
        if (starts.empty()) starts = st;
        msda_problem_t p;
        p.batch = bs;
        p.num_keys = static_cast<int32_t>(K >= 0 ? K : (sum < (int64_t(1) << 31) ? sum : -1));
        p.num_heads = M;
        p.embed_dims = D;
        p.num_levels = static_cast<int32_t>(shapes.size());
        p.num_points = P;
        p.num_queries = Q;
        p.dtype = static_cast<msda_dtype_t>(dtype);
        p.spatial_shapes = flat.data();
        p.level_start_index = starts.data();
        return p;
    }
};

const char* show(const msda_problem_t& p) {
    static char buf[256];
    snprintf(buf, sizeof buf, "bs %d K %d M %d D %d L %d P %d Q %d dtype %d", p.batch, p.num_keys, p.num_heads,
             p.embed_dims, p.num_levels, p.num_points, p.num_queries, static_cast<int>(p.dtype));
    return buf;
}

// Everything the launch code and the kernels assume of a valid descriptor.
void check_plan(const msda_problem_t& p) {
    using namespace msda_plan;
    const char* s = show(p);
    const msda::Problem pb = pack(&p);
    const int e = elem_bytes(p.dtype);
    // lane split: the group's active lanes cover the row exactly
    const LaneSplit ls = lane_split(p.embed_dims, p.dtype);
    EXPECT(ls.vecb == 4 || ls.vecb == 8 || ls.vecb == 16, "%s", s);
    EXPECT(ls.active * ls.vecb == p.embed_dims * e, "%s", s);
    EXPECT(ls.lpr >= 4 && ls.lpr <= 64 && (ls.lpr & (ls.lpr - 1)) == 0 && ls.lpr >= ls.active, "%s", s);
    EXPECT(pb.lpr_active == ls.active, "%s", s);
    // key segments: contiguous per level, 32..256 keys, a tile of at most 32 KB
    EXPECT(pb.seg_base[0] == 0, "%s", s);
    const int max_tile = pb.unit_records == msda::kSparseUnitRecords ? 16384 : 32768;
    int64_t nseg = 0;
    for (int l = 0; l < p.num_levels; ++l) {
        const int64_t hw = p.spatial_shapes[2 * l] * p.spatial_shapes[2 * l + 1];
        // at least 32 keys unless the tile bound allows fewer (16 keys of 256 floats in 16 KB), at most 256
        EXPECT(pb.seg_shift[l] >= 4 && pb.seg_shift[l] <= 8, "%s level %d shift %d", s, l, pb.seg_shift[l]);
        EXPECT(pb.seg_shift[l] >= 5 || (int64_t(32) * p.embed_dims * 4 > max_tile), "%s level %d", s, l);
        EXPECT((int64_t(1) << pb.seg_shift[l]) * p.embed_dims * 4 <= max_tile, "%s level %d", s, l);
        EXPECT(pb.lv.start[l] == p.level_start_index[l], "%s", s);
        if (nseg < kIndexLimit - 1) EXPECT(pb.seg_base[l] == nseg, "%s level %d", s, l);
        nseg += (hw + (int64_t(1) << pb.seg_shift[l]) - 1) >> pb.seg_shift[l];
    }
    EXPECT(pb.nseg == std::min<int64_t>(nseg, kIndexLimit - 1), "%s", s);
    EXPECT(pb.nplanes == p.batch * p.num_heads, "%s", s);
    // the record envelope
    const Layout lay = layout(&p, pb);
    if (lay.binned) {
        EXPECT(p.num_queries < (1 << msda::kQueryBits), "%s", s);
        EXPECT(pb.nseg <= msda::kMaxSegments, "%s", s);
        for (int l = 0; l < p.num_levels; ++l)
            EXPECT(p.spatial_shapes[2 * l] <= msda::kMaxBinnedExtent && p.spatial_shapes[2 * l + 1] <= msda::kMaxBinnedExtent,
                   "%s", s);
        EXPECT(max_records(&p) < kIndexLimit / 2, "%s", s);
        EXPECT(int64_t(pb.nplanes) * plane_records(&p) == max_records(&p), "%s", s);
        EXPECT(lay.max_units == int64_t(pb.nplanes) * plane_units(&p, pb), "%s", s);
        EXPECT(lay.max_units < kIndexLimit / 2, "%s", s);
        // every segment gets at least one unit; a segment of c records gets ceil(c / unit)
        EXPECT(plane_units(&p, pb) >= pb.nseg + (plane_records(&p) + pb.unit_records - 1) / pb.unit_records, "%s", s);
        // regions: in order, 256-byte aligned, each as large as its contents
        const int64_t nbins = int64_t(pb.nplanes) * pb.nseg;
        const size_t regions[] = {lay.counts, lay.cursor, lay.nunits, lay.multi, lay.units, lay.recs, lay.acc, lay.total};
        for (int i = 0; i + 1 < 8; ++i) EXPECT(regions[i] <= regions[i + 1] && regions[i] % 256 == 0, "%s region %d", s, i);
        if (!fused_count_scan(pb)) EXPECT(lay.cursor - lay.counts >= size_t(nbins * count_chunks(pb) * 4), "%s", s);
        EXPECT(lay.nunits - lay.cursor >= size_t(nbins * 4), "%s", s);
        EXPECT(lay.multi - lay.nunits >= size_t((3 * int64_t(pb.nplanes) + 1) * 4), "%s", s);
        EXPECT(lay.units - lay.multi >= size_t(nbins * 4), "%s", s);
        EXPECT(lay.recs - lay.units >= size_t(lay.max_units * 16), "%s", s);
        EXPECT(lay.acc - lay.recs >= size_t(max_records(&p) * 12), "%s", s);
        // counting: chunks cover the plane's samples, at most kMaxCountChunks rows
        const int64_t nsamp = int64_t(p.num_queries) * p.num_levels * p.num_points;
        if (!fused_count_scan(pb)) {
            EXPECT(count_chunk(pb) % 4 == 0, "%s", s);
            EXPECT(count_chunk(pb) * count_chunks(pb) >= nsamp, "%s", s);
            EXPECT(count_chunks(pb) <= msda::kMaxCountChunks, "%s", s);
        } else {
            EXPECT(nsamp <= msda::kCountScanSamples, "%s", s);
        }
    }
    if (p.dtype != MSDA_F32) EXPECT(lay.total - lay.acc >= size_t(value_elems(&p) * 4), "%s", s);
    // workgroup tiles: samples per gradient workgroup within its LDS records
    const int gpb = grad_tile(pb, ls.lpr);
    EXPECT(gpb >= 1 && gpb * ls.lpr <= msda::kBlock, "%s", s);
    EXPECT(int64_t(gpb) * p.num_levels * p.num_points <= msda::kMaxWgSamples, "%s", s);
    const int fgpb = tile_queries(pb, ls.lpr, 1024, true);
    EXPECT(fgpb >= 1 && fgpb * ls.lpr <= msda::kBlock, "%s", s);
    EXPECT(int64_t(fgpb) * p.num_levels * p.num_points <= 1024, "%s", s);
    // the backward's launches
    for (int acc = 0; acc < 2; ++acc) {
        const BackwardPlan b = plan_backward(&p, acc != 0);
        if (value_elems(&p) == 0) {
            EXPECT(b.zero_blocks == 0 && b.grad_blocks == 0 && b.accum_blocks == 0, "%s", s);
            continue;
        }
        if (sample_elems(&p) == 0) {
            EXPECT(b.grad_blocks == 0 && b.accum_blocks == 0 && b.count_blocks == 0 && b.scan_blocks == 0, "%s", s);
            EXPECT((b.zero_blocks > 0) == (acc == 0), "%s", s);
            continue;
        }
        EXPECT(b.binned == lay.binned, "%s", s);
        EXPECT(b.grad_blocks == plane_blocks(pb, gpb) && b.grad_blocks >= 1 && b.grad_blocks <= 0x7fffffff, "%s", s);
        // the accumulation reads the unit prefix that gradient workgroup 0 writes
        EXPECT(b.accum_blocks == 0 || b.grad_blocks >= 1, "%s", s);
        if (b.binned) {
            EXPECT(b.accum_blocks == lay.max_units && b.scan_blocks == pb.nplanes, "%s", s);
            EXPECT(b.zero_blocks == 0, "%s", s);
        } else {
            EXPECT(b.accum_blocks == 0 && b.count_blocks == 0 && b.scan_blocks == 0, "%s", s);
            EXPECT((b.zero_blocks > 0) == (acc == 0), "%s", s);
            // the pre-reduction's 16-bit entry ids: 4 corners per workgroup sample
            EXPECT(4 * int64_t(gpb) * p.num_levels * p.num_points <= 65536, "%s", s);
        }
        EXPECT((b.narrow_blocks > 0) == (acc == 0 && p.dtype != MSDA_F32), "%s", s);
    }
}

int status_of(Desc d) {
    msda_problem_t p = d.make();
    const int st = msda_plan::check_problem(&p);
    if (st == MSDA_SUCCESS) check_plan(p);
    return st;
}

}  // namespace

int main() {
    using msda_plan::check_problem;
    constexpr int OK = MSDA_SUCCESS, INVALID = MSDA_ERROR_INVALID_VALUE, UNSUPPORTED = MSDA_ERROR_NOT_SUPPORTED;
    // ---- fixed cases (the C-ABI host tests' descriptors) ----
    {
        Desc d;
        EXPECT(status_of(d) == OK, "default");
        for (int dt = 0; dt <= 4; ++dt) { Desc e; e.dtype = dt; EXPECT(status_of(e) == OK, "dtype %d", dt); }
        Desc a; a.D = 8; EXPECT(status_of(a) == OK, "D 8");
        Desc b; b.D = 256; EXPECT(status_of(b) == OK, "D 256");
        Desc c; c.M = 1; EXPECT(status_of(c) == OK, "M 1");
        Desc e; e.P = 16; EXPECT(status_of(e) == OK, "P 16");
        Desc f; f.shapes = {{1, 1}}; f.P = 64; EXPECT(status_of(f) == OK, "1x1 P 64");
        Desc g; g.bs = 0; EXPECT(status_of(g) == OK, "bs 0");
        Desc h; h.Q = 0; EXPECT(status_of(h) == OK, "Q 0");
        Desc i; i.shapes.assign(64, {3, 1}); i.P = 1; EXPECT(status_of(i) == OK, "64 levels");
    }
    {
        struct { int D, M, P, bs, Q, dtype; int64_t K; int code; } cases[] = {
            {12, 8, 4, 2, 300, 0, -1, UNSUPPORTED}, {264, 8, 4, 2, 300, 0, -1, UNSUPPORTED},
            {32, 9, 4, 2, 300, 0, -1, UNSUPPORTED}, {32, 8, 17, 2, 300, 0, -1, UNSUPPORTED},
            {0, 8, 4, 2, 300, 0, -1, INVALID},      {32, 0, 4, 2, 300, 0, -1, INVALID},
            {32, 8, 0, 2, 300, 0, -1, INVALID},     {32, 8, 4, -1, 300, 0, -1, INVALID},
            {32, 8, 4, 2, -3, 0, -1, INVALID},      {32, 8, 4, 2, 300, 7, -1, INVALID},
            {32, 8, 4, 2, 300, 5, -1, INVALID},     {32, 8, 4, 2, 300, 0, 17820, INVALID},
        };
        for (auto& c : cases) {
            Desc d;
            d.D = c.D; d.M = c.M; d.P = c.P; d.bs = c.bs; d.Q = c.Q; d.dtype = c.dtype; d.K = c.K;
            EXPECT(status_of(d) == c.code, "D %d M %d P %d bs %d Q %d dtype %d K %ld", c.D, c.M, c.P, c.bs, c.Q,
                   c.dtype, static_cast<long>(c.K));
        }
        Desc s1; s1.starts = {0, 13400, 16750, 17601}; EXPECT(status_of(s1) == INVALID, "starts");
        Desc s2; s2.starts = {1, 13401, 16751, 17601}; EXPECT(status_of(s2) == INVALID, "starts");
        Desc z; z.shapes = {{0, 5}}; z.K = 0; EXPECT(status_of(z) == INVALID, "H 0");
        Desc n; n.shapes = {{4, -2}}; n.K = 0; EXPECT(status_of(n) == INVALID, "W < 0");
        EXPECT(check_problem(nullptr) == INVALID, "null");
        Desc nn; msda_problem_t p = nn.make(); p.spatial_shapes = nullptr; EXPECT(check_problem(&p) == INVALID, "null shapes");
    }
    {   // 32-bit byte offsets per batch
        Desc a; a.shapes = {{4096, 2048}}; a.M = 8; a.D = 256; a.P = 1; a.Q = 1;
        EXPECT(status_of(a) == UNSUPPORTED, "value bytes");
        Desc b; b.shapes = {{4096, 2048}}; b.M = 1; b.D = 64; b.P = 1; b.Q = 1;
        EXPECT(status_of(b) == UNSUPPORTED, "2^31 bytes");
        b.dtype = 1; EXPECT(status_of(b) == OK, "fp16 2^30 bytes");
        Desc c; c.shapes = {{64, 64}}; c.M = 8; c.D = 256; c.P = 1; c.Q = 1 << 18;
        EXPECT(status_of(c) == UNSUPPORTED, "output bytes");
    }
    {   // record envelope edges: segments, query field, level extents
        Desc a; a.shapes = {{512, 1024}}; a.M = 2; a.D = 8; a.P = 4; a.Q = 2000; a.bs = 1;
        msda_problem_t p = a.make();
        EXPECT(status_of(a) == OK, "2048 segments");
        EXPECT(msda_plan::pack(&p).nseg == 2048 && msda_plan::layout(&p, msda_plan::pack(&p)).binned, "2048 binned");
        Desc b = a; b.shapes.push_back({2, 64}); b.starts.clear(); p = b.make();
        EXPECT(status_of(b) == OK && !msda_plan::layout(&p, msda_plan::pack(&p)).binned, "2052 atomic");
        Desc c = a; c.shapes.push_back({1, 1}); c.starts.clear(); p = c.make();
        EXPECT(status_of(c) == OK && !msda_plan::layout(&p, msda_plan::pack(&p)).binned, "2049 atomic");
        Desc q; q.shapes = {{64, 64}}; q.M = 1; q.D = 8; q.P = 1; q.bs = 1; q.Q = (1 << 24) - 1; p = q.make();
        EXPECT(status_of(q) == OK && msda_plan::layout(&p, msda_plan::pack(&p)).binned, "2^24-1 queries");
        q.Q = 1 << 24; p = q.make();
        EXPECT(status_of(q) == OK && !msda_plan::layout(&p, msda_plan::pack(&p)).binned, "2^24 queries");
        Desc w; w.shapes = {{2, 65534}}; w.M = 1; w.D = 8; w.P = 2; w.bs = 1; w.Q = 3000; p = w.make();
        EXPECT(status_of(w) == OK && msda_plan::layout(&p, msda_plan::pack(&p)).binned, "65534 wide");
        w.shapes = {{2, 65535}}; w.starts.clear(); p = w.make();
        EXPECT(status_of(w) == OK && !msda_plan::layout(&p, msda_plan::pack(&p)).binned, "65535 wide");
        Desc h; h.shapes = {{65534, 2}}; h.M = 1; h.D = 8; h.P = 2; h.bs = 1; h.Q = 3000; p = h.make();
        EXPECT(status_of(h) == OK && msda_plan::layout(&p, msda_plan::pack(&p)).binned, "65534 tall");
        Desc f; f.shapes = {{1, 600000}}; f.M = 1; f.D = 8; f.P = 1; f.bs = 1; f.Q = 64;
        EXPECT(status_of(f) == OK, "600000 wide");
    }
    // ---- seeded fuzz around the envelope ----
    std::mt19937_64 rng(20261203);
    auto pick = [&](std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); };
    const int n = 100000;
    int valid = 0;
    for (int it = 0; it < n; ++it) {
        Desc d;
        const int L = 1 + static_cast<int>(rng() % 8);
        d.P = static_cast<int>(pick({1, 2, 3, 4, 8, 16, 17, 64 / L, 64 / L + 1}));
        if (d.P < 1) d.P = 1;
        d.shapes.clear();
        for (int l = 0; l < L; ++l) {
            int64_t H = pick({1, 2, 3, 7, 13, 25, 64, 100, 134, 1024, 65534, 65535, int64_t(1 + rng() % 300)});
            int64_t W = pick({1, 2, 5, 17, 34, 67, 134, 128, 2048, 65534, 65535, int64_t(1 + rng() % 300)});
            d.shapes.push_back({H, W});
        }
        d.M = static_cast<int>(pick({1, 2, 4, 8, 9}));
        d.D = static_cast<int>(pick({8, 16, 24, 32, 64, 96, 128, 256, 12, 264}));
        d.Q = static_cast<int>(pick({0, 1, 16, 300, 900, 17821, (1 << 24) - 1, 1 << 24, int64_t(rng() % 100000)}));
        d.bs = static_cast<int>(pick({0, 1, 2, 4, 8}));
        d.dtype = static_cast<int>(pick({0, 1, 2, 3, 4, 0, 1, 2, 6}));
        int64_t sum = 0;
        for (auto& s : d.shapes) sum += s.first * s.second;
        if (sum >= (int64_t(1) << 31)) {
            d.K = 5;                         // any num_keys: the cumsum check rejects the descriptor first
        } else if (rng() % 16 == 0) {
            d.K = sum + 1;                   // inconsistent
        }
        const int st = status_of(d);
        EXPECT(st == OK || st == INVALID || st == UNSUPPORTED, "status %d", st);
        valid += st == OK;
    }
    printf("plan_fuzz ok: %d checks, %d fuzzed descriptors (%d valid)\n", g_checks, n, valid);
    return 0;
}
