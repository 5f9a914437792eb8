// Host planner: legal-plan enumeration, the MI355X prior that picks the
// automatic plan, validation of explicit plans, and the host replay of a
// plan's thread -> element mapping.
//
// Follows the solver structure of "TIRx Metal reduction lowering", section 6:
// legality is decided first (hard device limits and the register-stripe
// budget), the finite candidate set is enumerated exhaustively, a prior
// ranks the survivors, and an explicit plan is honoured exactly or rejected,
// never clamped.  The Metal cost prior itself is not used; the MI355X prior
// below is this library's own (wave64, 256 CUs x 4 SIMDs, VGPR-resident
// stripes), and measured plan choices for known shapes live in
// lr_plan_table.inc.
#include <algorithm>
#include <climits>
#include <cstring>

#include "lr_internal.hpp"
#include "lr_map.hpp"

namespace lr {

bool cache_chunks_compiled(int nch) {
    for (int i = 0; i < kNumCacheChunks; ++i)
        if (kCacheChunks[i] == nch) return true;
    return false;
}

static bool split_chunks_compiled(int nch) {
    for (int i = 0; i < kNumSplitChunks; ++i)
        if (kSplitChunks[i] == nch) return true;
    return false;
}

static int smallest_split_instance(int64_t need) {
    for (int i = 0; i < kNumSplitChunks; ++i)
        if (kSplitChunks[i] >= need) return kSplitChunks[i];
    return 0;
}

int64_t plan_workspace_bytes(const lr_plan& p, int64_t rows) {
    return p.family == LR_FAMILY_SPLIT && rows > 0 ? rows * (int64_t)p.splits * 2 * (int64_t)sizeof(float) : 0;
}

int64_t dispatch_rows(const lr_plan& p, int64_t rows) {
    const int64_t blocks = kMaxDispatchItems / std::max<int64_t>(1, p.threads_per_block);
    const int64_t per = p.family == LR_FAMILY_SPLIT ? blocks / std::max<int64_t>(1, p.splits)
                                                    : blocks * std::max<int64_t>(1, p.rows_per_block);
    return std::max<int64_t>(1, std::min(per, rows));
}

lr_plan piece_plan(const lr_plan& p, int64_t n) {
    lr_plan q = p;
    q.blocks = p.family == LR_FAMILY_SPLIT ? n * p.splits : (n + p.rows_per_block - 1) / p.rows_per_block;
    return q;
}

// 16-byte chunks a worker must reach for the widest row of the problem.
static int64_t max_row_chunks(int64_t cols, bool aligned) {
    return aligned ? cols / kVec : (cols + 3 + kVec - 1) / kVec;  // phase up to 3
}

// Fewest 16-byte chunks a row of the problem spans (phase 0).
static int64_t min_row_chunks(int64_t cols) { return (cols + kVec - 1) / kVec; }

// Chunks per lane a SPLIT plan needs: the longest segment over W = 64*S lanes.
static int64_t split_need(int64_t cols, bool aligned, int G, int S) {
    const int64_t L = (max_row_chunks(cols, aligned) + G - 1) / G;
    return (L + kWave * S - 1) / (kWave * S);
}

static int reductions_of(int op) {
    return (op == LR_OP_RMSNORM || op == LR_OP_ROW_SUM) ? 1 : 2;
}

static int smallest_cache_instance(int64_t need) {
    for (int i = 0; i < kNumCacheChunks; ++i)
        if (kCacheChunks[i] >= need) return kCacheChunks[i];
    return 0;
}

static bool narrow_chunks_compiled(int nch) {
    for (int i = 0; i < kNumNarrowChunks; ++i)
        if (kNarrowChunks[i] == nch) return true;
    return false;
}

static int smallest_lane_instance(int64_t need) {
    for (int i = 0; i < kNumLaneChunks; ++i)
        if (kLaneChunks[i] >= need) return kLaneChunks[i];
    return 0;
}

static int smallest_narrow_instance(int64_t need) {
    for (int i = 0; i < kNumNarrowChunks; ++i)
        if (kNarrowChunks[i] >= need) return kNarrowChunks[i];
    return 0;
}

// `lanes`: 4, 8, 16 or 32 for a CACHE plan of sub-wave teams (S = 1), else 0.
static lr_plan make_plan(int family, int S, int Q, int nch, int64_t rows, int64_t cols, int op, bool aligned,
                        int splits = 0, int lanes = 0) {
    lr_plan p;
    std::memset(&p, 0, sizeof(p));
    p.family = family;
    p.waves_per_row = S;
    p.rows_per_block = Q;
    p.vec = family == LR_FAMILY_ORDERED ? 1 : kVec;
    p.chunks_per_lane = nch;
    p.lanes_per_row = lanes != 0 ? lanes : kWave * S;
    p.threads_per_block = lanes != 0 ? lanes * Q : kWave * S * Q;
    p.splits = family == LR_FAMILY_SPLIT ? splits : 0;
    p.blocks = family == LR_FAMILY_SPLIT ? rows * splits : (rows + Q - 1) / Q;
    p.reductions = reductions_of(op);
    p.lds_bytes = family == LR_FAMILY_ORDERED ? (lanes == 1 ? kWave * (kVec * nch + 2) * 4 : Q * (kSlab + kTreeStack) * 4)
                  : family == LR_FAMILY_TREE  ? 2 * kMaxWaves * 4 + 2 * kMaxWaves * 128 * 4
                                              : 2 * kMaxWaves * 4;
    p.row_aligned = aligned ? 1 : 0;
    return p;
}

static bool valid_op(int op) { return op >= LR_OP_SOFTMAX && op <= LR_OP_ROW_MINMAX; }
static bool valid_policy(int p) { return p >= LR_UNORDERED_TREE && p <= LR_FOLD_RIGHT; }

// Families a policy may run on: unordered -> CACHE, STREAM, SPLIT; fold_left
// and fold_right -> ORDERED; ordered_tree -> TREE, ORDERED.
static bool family_allowed(int policy, int family) {
    switch (policy) {
        case LR_UNORDERED_TREE:
            return family == LR_FAMILY_CACHE || family == LR_FAMILY_STREAM || family == LR_FAMILY_SPLIT;
        case LR_ORDERED_TREE: return family == LR_FAMILY_TREE || family == LR_FAMILY_ORDERED;
        default: return family == LR_FAMILY_ORDERED;
    }
}

static lr_status check_problem(const lr_device_facts* f, int op, int64_t rows, int64_t cols, int policy) {
    if (f == nullptr) return LR_ERR_NULL_POINTER;
    if (!valid_op(op)) return LR_ERR_INVALID_ARGUMENT;
    if (!valid_policy(policy)) return LR_ERR_INVALID_POLICY;
    if (rows < 0 || cols < 1 || cols >= (int64_t(1) << 24) || rows > INT32_MAX) return LR_ERR_INVALID_SHAPE;
    if (f->compute_units < 1 || f->max_threads_per_block < kWave || f->wave_size != kWave)
        return LR_ERR_INVALID_ARGUMENT;
    return LR_OK;
}

lr_status validate_plan(const lr_device_facts* f, int op, int64_t rows, int64_t cols, int policy,
                        bool aligned, const lr_plan* p) {
    lr_status st = check_problem(f, op, rows, cols, policy);
    if (st != LR_OK) return st;
    if (p == nullptr) return LR_ERR_NULL_POINTER;
    const int S = p->waves_per_row, Q = p->rows_per_block, L = p->lanes_per_row;
    if (!family_allowed(policy, p->family)) return LR_ERR_UNREALIZABLE_PLAN;
    if (L == 1) {
        // one lane per row: ORDERED, one wavefront of 64 rows per workgroup
        // (the kernel's LDS tile holds exactly that), rows held in a compiled
        // register stripe of 4 * chunks_per_lane >= cols floats, any alignment
        if (p->family != LR_FAMILY_ORDERED || S != 1 || Q != kWave) return LR_ERR_UNREALIZABLE_PLAN;
        if (p->threads_per_block != Q || p->vec != 1 || p->splits != 0) return LR_ERR_UNREALIZABLE_PLAN;
        if (p->blocks != (rows + Q - 1) / Q || p->blocks > INT32_MAX) return LR_ERR_UNREALIZABLE_PLAN;
        bool compiled = false;
        for (int i = 0; i < kNumLaneChunks; ++i) compiled = compiled || kLaneChunks[i] == p->chunks_per_lane;
        if (!compiled || (int64_t)kVec * p->chunks_per_lane < cols) return LR_ERR_UNREALIZABLE_PLAN;
        return LR_OK;
    }
    if (narrow_lanes(L)) {
        // sub-wave teams: CACHE, or TREE with one chunk per lane on aligned
        // rows; one team per L lanes, whole waves per workgroup, a compiled
        // stripe that covers the widest row
        const bool tree = p->family == LR_FAMILY_TREE;
        if ((p->family != LR_FAMILY_CACHE && !tree) || S != 1 || Q < 1 || Q % (kWave / L) != 0)
            return LR_ERR_UNREALIZABLE_PLAN;
        if (tree && (!aligned || p->chunks_per_lane != 1)) return LR_ERR_UNREALIZABLE_PLAN;
        if ((int64_t)L * Q > f->max_threads_per_block || p->threads_per_block != L * Q) return LR_ERR_UNREALIZABLE_PLAN;
        if (p->splits != 0 || p->blocks != (rows + Q - 1) / Q || p->blocks > INT32_MAX) return LR_ERR_UNREALIZABLE_PLAN;
        if (p->vec != kVec || !narrow_chunks_compiled(p->chunks_per_lane)) return LR_ERR_UNREALIZABLE_PLAN;
        if (p->chunks_per_lane < (max_row_chunks(cols, aligned) + L - 1) / L) return LR_ERR_UNREALIZABLE_PLAN;
        return LR_OK;
    }
    if (S < 1 || Q < 1 || S > kMaxWaves || Q > kMaxWaves || S * Q > kMaxWaves) return LR_ERR_UNREALIZABLE_PLAN;
    if (L != 0 && L != kWave * S) return LR_ERR_UNREALIZABLE_PLAN;  // 0: whole waves
    if (p->threads_per_block != kWave * S * Q || p->threads_per_block > f->max_threads_per_block)
        return LR_ERR_UNREALIZABLE_PLAN;
    if (p->family == LR_FAMILY_SPLIT) {
        // one segment per workgroup; every lane of a merging wave holds one
        // partial, and no row has fewer chunks than segments
        const int G = p->splits;
        if (Q != 1 || G < 2 || G > kMaxSplits || G > min_row_chunks(cols)) return LR_ERR_UNREALIZABLE_PLAN;
        if (p->blocks != rows * G || p->blocks > INT32_MAX) return LR_ERR_UNREALIZABLE_PLAN;
        if (p->vec != kVec || !split_chunks_compiled(p->chunks_per_lane)) return LR_ERR_UNREALIZABLE_PLAN;
        if (p->chunks_per_lane < split_need(cols, aligned, G, S)) return LR_ERR_UNREALIZABLE_PLAN;
        return LR_OK;
    }
    const int64_t blocks = (rows + Q - 1) / Q;
    if (p->splits != 0 || p->blocks != blocks || blocks > INT32_MAX) return LR_ERR_UNREALIZABLE_PLAN;
    switch (p->family) {
        case LR_FAMILY_TREE:
            // the cache layout with aligned rows; at most 128 slabs of 256 floats
            if (!aligned || cols > kTreeMaxCols) return LR_ERR_UNREALIZABLE_PLAN;
            [[fallthrough]];
        case LR_FAMILY_CACHE: {
            if (p->vec != kVec || !cache_chunks_compiled(p->chunks_per_lane)) return LR_ERR_UNREALIZABLE_PLAN;
            const int64_t need = (max_row_chunks(cols, aligned) + kWave * S - 1) / (kWave * S);
            if (p->chunks_per_lane < need) return LR_ERR_UNREALIZABLE_PLAN;
            if (p->threads_per_block > cache_max_threads(p->chunks_per_lane)) return LR_ERR_UNREALIZABLE_PLAN;
            return LR_OK;
        }
        case LR_FAMILY_STREAM:
            if (p->vec != kVec || p->chunks_per_lane != kStreamUnroll) return LR_ERR_UNREALIZABLE_PLAN;
            return LR_OK;
        case LR_FAMILY_ORDERED:
            if (S != 1 || p->vec != 1 || p->chunks_per_lane != 0) return LR_ERR_UNREALIZABLE_PLAN;
            return LR_OK;
        default:
            return LR_ERR_UNREALIZABLE_PLAN;
    }
}

// All legal plans in enumeration order: family, then S, then Q.
static int enumerate_all(const lr_device_facts* f, int op, int64_t rows, int64_t cols, int policy,
                         bool aligned, lr_plan* out, int cap) {
    int n = 0;
    auto push = [&](const lr_plan& p) {
        if (validate_plan(f, op, rows, cols, policy, aligned, &p) != LR_OK) return;
        if (out != nullptr && n < cap) out[n] = p;
        ++n;
    };
    const int64_t nv = max_row_chunks(cols, aligned);
    if (policy != LR_UNORDERED_TREE) {
        if (policy == LR_ORDERED_TREE) {
            for (int S = 1; S <= kMaxWaves; ++S) {
                const int nch = smallest_cache_instance((nv + kWave * S - 1) / (kWave * S));
                if (nch == 0) continue;
                for (int Q = 1; S * Q <= kMaxWaves; ++Q)
                    push(make_plan(LR_FAMILY_TREE, S, Q, nch, rows, cols, op, aligned));
            }
            for (int L : kNarrowLanes) {  // sub-wave teams, one chunk per lane
                if (nv > L) continue;
                for (int w = 1; w <= kMaxWaves; ++w)
                    push(make_plan(LR_FAMILY_TREE, 1, w * (kWave / L), 1, rows, cols, op, aligned, 0, L));
            }
        }
        for (int Q = 1; Q <= kMaxWaves; ++Q) push(make_plan(LR_FAMILY_ORDERED, 1, Q, 0, rows, cols, op, aligned));
        // one lane per row: narrow rows, one wavefront per workgroup
        {
            const int n4 = smallest_lane_instance((cols + kVec - 1) / kVec);
            if (n4 != 0) push(make_plan(LR_FAMILY_ORDERED, 1, kWave, n4, rows, cols, op, aligned, 0, 1));
        }
        return n;
    }
    for (int S = 1; S <= kMaxWaves; ++S) {
        const int64_t need = (nv + kWave * S - 1) / (kWave * S);
        const int nch = smallest_cache_instance(need);
        if (nch == 0) continue;
        for (int Q = 1; S * Q <= kMaxWaves; ++Q) push(make_plan(LR_FAMILY_CACHE, S, Q, nch, rows, cols, op, aligned));
    }
    // sub-wave teams for narrow rows: L lanes per row, 1 .. 16 waves per workgroup
    for (int L : kNarrowLanes) {
        const int nch = smallest_narrow_instance((nv + L - 1) / L);
        if (nch == 0) continue;
        for (int w = 1; w <= kMaxWaves; ++w)
            push(make_plan(LR_FAMILY_CACHE, 1, w * (kWave / L), nch, rows, cols, op, aligned, 0, L));
    }
    for (int S = 1; S <= kMaxWaves; ++S)
        for (int Q = 1; S * Q <= kMaxWaves; ++Q)
            push(make_plan(LR_FAMILY_STREAM, S, Q, kStreamUnroll, rows, cols, op, aligned));
    for (int G = 2; G <= kMaxSplits && G <= min_row_chunks(cols); G *= 2)
        for (int S = 1; S <= kMaxWaves; ++S) {
            const int nch = smallest_split_instance(split_need(cols, aligned, G, S));
            if (nch != 0) push(make_plan(LR_FAMILY_SPLIT, S, 1, nch, rows, cols, op, aligned, G));
        }
    return n;
}

// ---------------------------------------------------------------------------
// MI355X prior.  Rows are independent and the kernels are HBM-bound, so the
// plan's job is to keep enough 128-bit loads in flight on every CU while
// keeping the register stripe short:
//   * enough wavefronts: the smallest S with rows*S >= 2 waves per SIMD of
//     the device, so few-row problems spread each row over more waves;
//   * register budget: widen S until the stripe is <= 8 chunks (32 floats)
//     per lane -- short stripes keep occupancy high and leave registers for
//     the gamma/beta prefetch;
//   * cross-entropy keeps nothing after its single pass, so long rows take
//     the STREAM family (online max / sum of exp, no register copy);
//   * one row per workgroup (on MI355X, packing four single-wave rows per
//     workgroup measured up to 10% slower: LayerNorm 65536 x 256, 23.7 against
//     26.1 us);
//   * rows of at most 32 chunks, when rows are plentiful: sub-wave teams, one
//     chunk per lane, one wave per workgroup for 16-byte aligned rows and
//     four for misaligned ones (softmax 262144 x 64: 22.0 against 50.8 us for
//     whole waves; 262144 x 50: 22.3 against 24.4 us with one wave).
// Measured winners for known shapes (lr_plan_table.inc) take precedence.
// ---------------------------------------------------------------------------
struct TableEntry {
    int op;
    int policy;
    int64_t rows;
    int64_t cols;
    int aligned;
    int family, S, Q, nch;
    int splits;  // SPLIT entries only
    int lanes;   // sub-wave CACHE entries only (0: whole waves)
    int without_params;  // 1: only for a norm called without gamma and beta
};

static const TableEntry kTable[] = {
#include "lr_plan_table.inc"
};

// Rows too few to fill the device, when a workspace is available: G
// segments per row, G the smallest power of two with rows*G >= the CU count,
// halved while a segment would hold fewer than 256 chunks (1024 floats: the
// second launch has to pay for itself); S the fewest waves with a stripe of
// at most 4 chunks per lane.  G < 2 means: do not split.  Only the fused
// residual LayerNorm splits (three tensor streams per row): on MI355X at
// 64 x 12288 in a graph, 5.1 us split against 5.6 us in one launch.  The
// other ops finish faster in one launch than any split plan (LayerNorm
// 64 x 12288 3.9 us, 64 x 12289 5.6 us; the split plans 4.7 and 6.2 us).
static lr_plan split_prior(const lr_device_facts* f, int op, int64_t rows, int64_t cols, bool aligned) {
    lr_plan none;
    std::memset(&none, 0, sizeof(none));
    const int64_t cus = f->compute_units;
    if (op != LR_OP_ADD_LAYERNORM) return none;
    if (rows < 1 || 2 * rows > cus) return none;
    int G = 1;
    while (G < kMaxSplits && rows * G < cus) G *= 2;
    while (G >= 2 && min_row_chunks(cols) / G < 256) G /= 2;
    if (G < 2) return none;
    int S = 1;
    while (S < kMaxWaves && split_need(cols, aligned, G, S) > 4) ++S;
    const int nch = smallest_split_instance(split_need(cols, aligned, G, S));
    if (nch == 0) return none;
    return make_plan(LR_FAMILY_SPLIT, S, 1, nch, rows, cols, op, aligned, G);
}

static lr_plan prior_plan(const lr_device_facts* f, int op, int64_t rows, int64_t cols, int policy,
                          bool aligned, bool allow_split, bool params) {
    auto matches = [&](const TableEntry& e) {
        return e.op == op && e.policy == policy && e.rows == rows && e.cols == cols &&
               e.aligned == (aligned ? 1 : 0) && (e.without_params == 0 || !params);
    };
    auto from_entry = [&](const TableEntry& e) {
        return make_plan(e.family, e.S, e.Q, e.nch, rows, cols, op, aligned, e.splits, e.lanes);
    };
    if (allow_split && policy == LR_UNORDERED_TREE) {
        // a measured SPLIT winner; else the split prior, unless a measured
        // workspace-free winner is listed for the shape
        bool listed = false;
        for (const TableEntry& e : kTable) {
            if (!matches(e)) continue;
            if (e.family != LR_FAMILY_SPLIT) {
                listed = true;
                continue;
            }
            lr_plan p = from_entry(e);
            if (validate_plan(f, op, rows, cols, policy, aligned, &p) == LR_OK) return p;
        }
        if (!listed) {
            lr_plan p = split_prior(f, op, rows, cols, aligned);
            if (p.family == LR_FAMILY_SPLIT && validate_plan(f, op, rows, cols, policy, aligned, &p) == LR_OK)
                return p;
        }
    }
    for (const TableEntry& e : kTable) {
        if (!matches(e) || e.family == LR_FAMILY_SPLIT) continue;
        lr_plan p = from_entry(e);
        if (validate_plan(f, op, rows, cols, policy, aligned, &p) == LR_OK) return p;
    }
    const int64_t simds = (int64_t)f->compute_units * (f->simds_per_cu > 0 ? f->simds_per_cu : 4);
    const int64_t nv = max_row_chunks(cols, aligned);
    const int64_t target_waves = 2 * simds;
    auto need = [&](int s) { return (nv + kWave * s - 1) / (kWave * s); };
    int S = 1;
    while (S < kMaxWaves && (int64_t)rows * S < target_waves) ++S;
    while (S < kMaxWaves && need(S) > 8) ++S;
    if (policy != LR_UNORDERED_TREE) {
        // ordered_tree on aligned rows: the cache layout with the tree combine
        // (sub-wave teams for narrow rows, as for the unordered policy)
        if (policy == LR_ORDERED_TREE) {
            if (S == 1 && nv <= 32) {
                int L = 4;
                while (L < nv) L *= 2;
                lr_plan p = make_plan(LR_FAMILY_TREE, 1, kWave / L, 1, rows, cols, op, aligned, 0, L);
                if (validate_plan(f, op, rows, cols, policy, aligned, &p) == LR_OK) return p;
            }
            lr_plan p = make_plan(LR_FAMILY_TREE, S, 1, smallest_cache_instance(need(S)), rows, cols, op, aligned);
            if (validate_plan(f, op, rows, cols, policy, aligned, &p) == LR_OK) return p;
        }
        // the folds (and the tree on misaligned rows): rows plentiful and at
        // most 64 floats wide take one lane per row (on MI355X: RMSNorm
        // 262144 x 64 26 us against 124 us one wave per row, 262144 x 50 23
        // against 123 us, cross-entropy 262144 x 32 9 against 104 us,
        // softmax 1048576 x 16 25 against 848 us); wider rows one wave per row
        if (S == 1 && cols <= kVec * kLaneChunks[kNumLaneChunks - 1]) {
            const int n4 = smallest_lane_instance((cols + kVec - 1) / kVec);
            lr_plan p = make_plan(LR_FAMILY_ORDERED, 1, kWave, n4, rows, cols, op, aligned, 0, 1);
            if (n4 != 0 && validate_plan(f, op, rows, cols, policy, aligned, &p) == LR_OK) return p;
        }
        const int Q = rows >= 4 * simds ? 4 : 1;
        return make_plan(LR_FAMILY_ORDERED, 1, Q, 0, rows, cols, op, aligned);
    }
    if (S == 1 && nv <= 32) {
        // rows plentiful and narrow: sub-wave teams with one chunk per lane
        // (the smallest power of two lanes from 4 to 32 that covers the row)
        int L = 4;
        while (L < nv) L *= 2;
        // one wave per workgroup on aligned rows, four on misaligned rows and
        // for cross-entropy (on MI355X: 262144 x 32 10.1 us against 10.6,
        // 1048576 x 16 18.6 against 19.0)
        const int waves = aligned && op != LR_OP_CROSS_ENTROPY ? 1 : 4;
        lr_plan p = make_plan(LR_FAMILY_CACHE, 1, waves * (kWave / L), 1, rows, cols, op, aligned, 0, L);
        if (validate_plan(f, op, rows, cols, policy, aligned, &p) == LR_OK) return p;
    }
    int family = LR_FAMILY_CACHE;
    int nch = smallest_cache_instance(need(S));
    if (nch == 0 || (op == LR_OP_CROSS_ENTROPY && need(S) > 8)) {
        family = LR_FAMILY_STREAM;
        nch = kStreamUnroll;
        if (op == LR_OP_CROSS_ENTROPY) S = std::max(S, 8);
    }
    lr_plan p = make_plan(family, S, 1, nch, rows, cols, op, aligned);
    if (validate_plan(f, op, rows, cols, policy, aligned, &p) != LR_OK)
        p = make_plan(LR_FAMILY_STREAM, S, 1, kStreamUnroll, rows, cols, op, aligned);
    return p;
}

}  // namespace lr

using namespace lr;

extern "C" void lr_device_facts_mi355x(lr_device_facts* out) {
    if (out == nullptr) return;
    out->compute_units = 256;
    out->max_threads_per_block = 1024;
    out->simds_per_cu = 4;
    out->wave_size = 64;
}

namespace lr {

lr_status plan_for_call(const lr_device_facts* facts, int op, int64_t rows, int64_t cols, int policy,
                        bool row_aligned, bool allow_split, bool params, lr_plan* out) {
    lr_status st = check_problem(facts, op, rows, cols, policy);
    if (st != LR_OK) return st;
    if (out == nullptr) return LR_ERR_NULL_POINTER;
    const bool aligned = row_aligned && cols % kVec == 0;
    lr_plan p = prior_plan(facts, op, rows, cols, policy, aligned, allow_split, params);
    st = validate_plan(facts, op, rows, cols, policy, aligned, &p);
    if (st != LR_OK) return st;
    *out = p;
    return LR_OK;
}

}  // namespace lr

extern "C" lr_status lr_plan_for_device(const lr_device_facts* facts, lr_op op, int64_t rows, int64_t cols,
                                        lr_reduction_policy policy, int32_t row_aligned, lr_plan* out) {
    lr_status st = check_problem(facts, op, rows, cols, policy);
    if (st != LR_OK) return st;
    if (out == nullptr) return LR_ERR_NULL_POINTER;
    const bool aligned = row_aligned != 0 && cols % kVec == 0;
    lr_plan p = prior_plan(facts, op, rows, cols, policy, aligned, false, true);
    st = validate_plan(facts, op, rows, cols, policy, aligned, &p);
    if (st != LR_OK) return st;
    *out = p;
    return LR_OK;
}

extern "C" lr_status lr_plan_for_device_ws(const lr_device_facts* facts, lr_op op, int64_t rows, int64_t cols,
                                           lr_reduction_policy policy, int32_t row_aligned, lr_plan* out) {
    lr_status st = check_problem(facts, op, rows, cols, policy);
    if (st != LR_OK) return st;
    if (out == nullptr) return LR_ERR_NULL_POINTER;
    const bool aligned = row_aligned != 0 && cols % kVec == 0;
    lr_plan p = prior_plan(facts, op, rows, cols, policy, aligned, true, true);
    st = validate_plan(facts, op, rows, cols, policy, aligned, &p);
    if (st != LR_OK) return st;
    *out = p;
    return LR_OK;
}

extern "C" uint64_t lr_plan_workspace_bytes(const lr_plan* plan, int64_t rows) {
    return plan == nullptr ? 0 : (uint64_t)plan_workspace_bytes(*plan, rows);
}

extern "C" int64_t lr_dispatch_rows(const lr_plan* plan, int64_t rows) {
    return plan == nullptr || rows < 1 ? 0 : dispatch_rows(*plan, rows);
}

extern "C" lr_status lr_plan_enumerate(const lr_device_facts* facts, lr_op op, int64_t rows, int64_t cols,
                                       lr_reduction_policy policy, int32_t row_aligned, lr_plan* out,
                                       int32_t capacity, int32_t* count) {
    lr_status st = check_problem(facts, op, rows, cols, policy);
    if (st != LR_OK) return st;
    if (count == nullptr || capacity < 0 || (out == nullptr && capacity > 0)) return LR_ERR_NULL_POINTER;
    const bool aligned = row_aligned != 0 && cols % kVec == 0;
    *count = enumerate_all(facts, op, rows, cols, policy, aligned, out, capacity);
    return LR_OK;
}

extern "C" lr_status lr_plan_validate(const lr_device_facts* facts, lr_op op, int64_t rows, int64_t cols,
                                      lr_reduction_policy policy, int32_t row_aligned, const lr_plan* plan) {
    const bool aligned = row_aligned != 0 && cols % kVec == 0;
    return validate_plan(facts, op, rows, cols, policy, aligned, plan);
}

extern "C" lr_status lr_coverage_check(const lr_plan* p, int64_t rows, int64_t cols, int32_t phase,
                                       uint32_t* counts) {
    if (p == nullptr || counts == nullptr) return LR_ERR_NULL_POINTER;
    if (rows < 0 || cols < 1 || cols >= (int64_t(1) << 24)) return LR_ERR_INVALID_SHAPE;
    if (phase < 0 || phase > 3) return LR_ERR_INVALID_ARGUMENT;
    const int S = p->waves_per_row, Q = p->rows_per_block, L = p->lanes_per_row;
    const bool narrow = narrow_lanes(L);
    if (L == 1) {
        // one lane per row: lane tid of block b owns row b * Q + tid, every element
        if (p->family != LR_FAMILY_ORDERED || S != 1 || Q < 1 || p->threads_per_block != Q)
            return LR_ERR_UNREALIZABLE_PLAN;
        for (int64_t b = 0; b < p->blocks; ++b)
            for (int tid = 0; tid < Q; ++tid) {
                const int64_t row = b * Q + tid;
                if (row >= rows) continue;
                for (int j = 0; j < kVec * p->chunks_per_lane && j < cols; ++j) counts[row * cols + j] += 1;
            }
        return LR_OK;
    }
    if (S < 1 || Q < 1 || p->threads_per_block != (narrow ? L * Q : kWave * S * Q)) return LR_ERR_UNREALIZABLE_PLAN;
    if (narrow && ((p->family != LR_FAMILY_CACHE && p->family != LR_FAMILY_TREE) || S != 1))
        return LR_ERR_UNREALIZABLE_PLAN;
    const int c = (int)cols;
    if (p->family == LR_FAMILY_SPLIT && (p->splits < 1 || Q != 1)) return LR_ERR_UNREALIZABLE_PLAN;
    for (int64_t b = 0; b < p->blocks; ++b) {
        for (int tid = 0; tid < p->threads_per_block; ++tid) {
            if (p->family == LR_FAMILY_SPLIT) {
                // block b holds segment b % G of row b / G (workers w + W*i)
                const Team t = team_of(tid, S);
                const int W = kWave * S;
                const int64_t row = b / p->splits;
                if (row >= rows) continue;
                const int h = (int)((phase + (row * cols) % kVec) % kVec);
                const int nv = chunks_of(h, c);
                const SegmentBounds sb = segment_bounds(nv, p->splits, (int)(b % p->splits));
                for (int i = 0; i < p->chunks_per_lane; ++i) {
                    const int k = sb.k0 + chunk_index(t.w, W, i);
                    if (k >= sb.k1) continue;
                    for (int j = 0; j < kVec; ++j) {
                        const int e = elem_index(k, j, h);
                        if (elem_valid(e, c)) counts[row * cols + e] += 1;
                    }
                }
                continue;
            }
            if (p->family == LR_FAMILY_ORDERED) {
                const int lane = tid % kWave, wave = tid / kWave;
                const int64_t row = row_of(b, Q, wave);
                if (row >= rows) continue;
                for (int slab = 0; slab * kSlab < c; ++slab)
                    for (int i = 0; i < kSlab / kWave; ++i) {
                        const int e = ordered_elem(slab, i, lane);
                        if (e < c) counts[row * cols + e] += 1;
                    }
                continue;
            }
            const Team t = narrow ? team_of_group(tid / kWave, tid % kWave, L) : team_of(tid, S);
            const int W = narrow ? L : kWave * S;
            const int64_t row = row_of(b, Q, t.q);
            if (row >= rows) continue;
            const int h = (int)((phase + (row * cols) % kVec) % kVec);
            const int nv = chunks_of(h, c);
            auto visit = [&](int k) {
                if (k >= nv) return;
                for (int j = 0; j < kVec; ++j) {
                    const int e = elem_index(k, j, h);
                    if (elem_valid(e, c)) counts[row * cols + e] += 1;
                }
            };
            if (p->family == LR_FAMILY_CACHE || p->family == LR_FAMILY_TREE) {
                for (int cc = 0; cc < p->chunks_per_lane; ++cc) visit(chunk_index(t.w, W, cc));
            } else {
                const int U = p->chunks_per_lane;
                for (int k0 = t.w; k0 < nv; k0 += W * U)
                    for (int u = 0; u < U; ++u) visit(k0 + W * u);
            }
        }
    }
    return LR_OK;
}
