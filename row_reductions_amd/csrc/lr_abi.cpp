// C-ABI entry points of liblr.so: argument validation (before any HIP
// call), plan selection, kernel dispatch and status mapping.  Declarations
// and the full contract are in include/lr.h.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "lr_internal.hpp"
#include "lr_map.hpp"

namespace lr {

lr_status validate_plan(const lr_device_facts* f, int op, int64_t rows, int64_t cols, int policy,
                        bool aligned, const lr_plan* p);
// The automatic plan of a call (lr_planner.cpp): lr_plan_for_device, or with
// allow_split the plan of lr_plan_for_device_ws, where `params` says whether
// a norm's call gives gamma or beta; without them a norm may take a plan the
// table lists for that case.
lr_status plan_for_call(const lr_device_facts* facts, int op, int64_t rows, int64_t cols, int policy,
                        bool row_aligned, bool allow_split, bool params, lr_plan* out);

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_facts_mu;
bool g_facts_ok[kMaxDevices];
lr_device_facts g_facts[kMaxDevices];

lr_status current_facts(lr_device_facts* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LR_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_facts_mu);
    if (!g_facts_ok[dev]) {
        int cus = 0, maxt = 0, ws = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&maxt, hipDeviceAttributeMaxThreadsPerBlock, dev) != hipSuccess ||
            hipDeviceGetAttribute(&ws, hipDeviceAttributeWarpSize, dev) != hipSuccess)
            return LR_ERR_HIP;
        lr_device_facts f;
        f.compute_units = cus;
        f.max_threads_per_block = maxt;
        f.simds_per_cu = 4;
        f.wave_size = ws;
        g_facts[dev] = f;
        g_facts_ok[dev] = true;
    }
    *out = g_facts[dev];
    return LR_OK;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Call {
    int op;
    const float* x;
    const float* gamma;
    const float* beta;
    float* y;
    const int64_t* labels;
    float* losses;
    int64_t rows;
    int64_t cols;
    float eps;
    int policy;
    const float* residual = nullptr;  // fused residual LayerNorm
    float* sum_out = nullptr;         // fused residual LayerNorm, optional
    float* sums = nullptr;            // row sum
    float* mins = nullptr;            // row minimum, optional
    float* maxs = nullptr;            // row maximum, optional
    void* workspace = nullptr;        // split family partials (lr_run_f32)
    uint64_t workspace_bytes = 0;
};

lr_status validate_call(const Call& c) {
    if (c.policy < LR_UNORDERED_TREE || c.policy > LR_FOLD_RIGHT) return LR_ERR_INVALID_POLICY;
    const bool ce = c.op == LR_OP_CROSS_ENTROPY;
    const bool res = c.op == LR_OP_ADD_LAYERNORM;
    const bool per_row = ce || c.op == LR_OP_ROW_SUM || c.op == LR_OP_ROW_MINMAX;  // one value per row out
    if (c.x == nullptr) return LR_ERR_NULL_POINTER;
    if (ce && (c.labels == nullptr || c.losses == nullptr)) return LR_ERR_NULL_POINTER;
    if (c.op == LR_OP_ROW_SUM && c.sums == nullptr) return LR_ERR_NULL_POINTER;
    if (c.op == LR_OP_ROW_MINMAX && c.mins == nullptr && c.maxs == nullptr) return LR_ERR_NULL_POINTER;
    if (!per_row && c.y == nullptr) return LR_ERR_NULL_POINTER;
    if (res && c.residual == nullptr) return LR_ERR_NULL_POINTER;
    if (c.rows < 0 || c.cols < 1 || c.cols >= (int64_t(1) << 24) || c.rows > INT32_MAX) return LR_ERR_INVALID_SHAPE;
    if (c.rows > INT64_MAX / 4 / c.cols) return LR_ERR_INVALID_SHAPE;
    if (c.op == LR_OP_RMSNORM || c.op == LR_OP_LAYERNORM || res) {
        if (!std::isfinite(c.eps) || c.eps < 0.0f) return LR_ERR_INVALID_EPS;
    }
    auto a4 = [](const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
    if (!a4(c.x) || !a4(c.y) || !a4(c.gamma) || !a4(c.beta) || !a4(c.losses) || !a4(c.residual) ||
        !a4(c.sum_out) || !a4(c.sums) || !a4(c.mins) || !a4(c.maxs))
        return LR_ERR_MISALIGNED;
    if (c.labels != nullptr && (reinterpret_cast<uintptr_t>(c.labels) & 7u) != 0) return LR_ERR_MISALIGNED;
    const int64_t tb = c.rows * c.cols * 4;
    const Range rx = range_of(c.x, tb);
    if (ce) {
        const Range rl = range_of(c.losses, c.rows * 4), rlab = range_of(c.labels, c.rows * 8);
        if (c.rows > 0 && (overlap(rl, rx) || overlap(rl, rlab))) return LR_ERR_ALIASING;
    } else if (per_row) {
        const float* outs[3] = {c.sums, c.mins, c.maxs};
        for (int i = 0; i < 3 && c.rows > 0; ++i) {
            if (outs[i] == nullptr) continue;
            const Range ro = range_of(outs[i], c.rows * 4);
            if (overlap(ro, rx)) return LR_ERR_ALIASING;
            for (int j = i + 1; j < 3; ++j)
                if (outs[j] != nullptr && overlap(ro, range_of(outs[j], c.rows * 4))) return LR_ERR_ALIASING;
        }
    } else if (c.rows > 0) {
        // an output may be exactly one of the row inputs (in place); any other
        // overlap with an input, or between the two outputs, is rejected
        auto apart_or_same = [&](const float* o, const float* in) {
            return o == in || !overlap(range_of(o, tb), range_of(in, tb));
        };
        auto output_ok = [&](const float* o) {
            const Range ro = range_of(o, tb);
            if (!apart_or_same(o, c.x)) return false;
            if (res && !apart_or_same(o, c.residual)) return false;
            if (c.gamma != nullptr && overlap(ro, range_of(c.gamma, c.cols * 4))) return false;
            if (c.beta != nullptr && overlap(ro, range_of(c.beta, c.cols * 4))) return false;
            return true;
        };
        if (!output_ok(c.y)) return LR_ERR_ALIASING;
        if (c.sum_out != nullptr && (!output_ok(c.sum_out) || overlap(range_of(c.sum_out, tb), range_of(c.y, tb))))
            return LR_ERR_ALIASING;
    }
    if (c.workspace == nullptr && c.workspace_bytes > 0) return LR_ERR_NULL_POINTER;
    if (c.workspace != nullptr && c.workspace_bytes > 0 && c.rows > 0) {
        if (!aligned16(c.workspace)) return LR_ERR_MISALIGNED;
        if (c.workspace_bytes > (uint64_t)INT64_MAX) return LR_ERR_INVALID_ARGUMENT;
        // the workspace overlaps no tensor of the call
        const Range rw = range_of(c.workspace, (int64_t)c.workspace_bytes);
        const int64_t vb = c.cols * 4, ob = c.rows * 4;
        const struct {
            const void* p;
            int64_t bytes;
        } all[] = {{c.x, tb},          {c.residual, tb}, {c.y, tb},    {c.sum_out, tb}, {c.gamma, vb},
                   {c.beta, vb},       {c.labels, c.rows * 8},         {c.losses, ob},  {c.sums, ob},
                   {c.mins, ob},       {c.maxs, ob}};
        for (const auto& t : all)
            if (t.p != nullptr && overlap(rw, range_of(t.p, t.bytes))) return LR_ERR_ALIASING;
    }
    return LR_OK;
}

hipError_t launch_piece(int op, int policy, const KArgs& a, const lr_plan& plan, bool aligned, hipStream_t stream) {
    if (plan.family == LR_FAMILY_ORDERED) {
        return plan.lanes_per_row == 1 ? launch_ordered_lane(op, policy, a, plan, stream)
                                       : launch_ordered(op, policy, a, plan, stream);
    }
    if (plan.family == LR_FAMILY_TREE) {
        switch (op) {
            case LR_OP_SOFTMAX: return launch_tree_softmax(a, plan, aligned, stream);
            case LR_OP_RMSNORM: return launch_tree_rmsnorm(a, plan, aligned, stream);
            case LR_OP_LAYERNORM: return launch_tree_layernorm(a, plan, aligned, stream);
            case LR_OP_ADD_LAYERNORM: return launch_tree_add_layernorm(a, plan, aligned, stream);
            case LR_OP_ROW_SUM: return launch_tree_row_sum(a, plan, aligned, stream);
            case LR_OP_ROW_MINMAX: return launch_tree_row_minmax(a, plan, aligned, stream);
            default: return launch_tree_cross_entropy(a, plan, aligned, stream);
        }
    }
    switch (op) {
        case LR_OP_SOFTMAX: return launch_softmax(a, plan, aligned, stream);
        case LR_OP_RMSNORM: return launch_rmsnorm(a, plan, aligned, stream);
        case LR_OP_LAYERNORM: return launch_layernorm(a, plan, aligned, stream);
        case LR_OP_ADD_LAYERNORM: return launch_add_layernorm(a, plan, aligned, stream);
        case LR_OP_ROW_SUM: return launch_row_sum(a, plan, aligned, stream);
        case LR_OP_ROW_MINMAX: return launch_row_minmax(a, plan, aligned, stream);
        default: return launch_cross_entropy(a, plan, aligned, stream);
    }
}

// Arguments of the row piece [r0, r0 + n): every row pointer advanced by r0
// rows.  A row's 16-byte phase is read from its own address and the
// same-phase flags compare two row pointers advanced alike, so both carry
// over.  The split workspace is not advanced: pieces run one after another on
// one stream and each needs no more of it than the whole call.
KArgs piece_args(const KArgs& a, int64_t r0, int64_t n, bool per_row) {
    auto adv = [](auto* p, int64_t k) { return p == nullptr ? p : p + k; };
    const int64_t e0 = r0 * a.cols;
    KArgs b = a;
    b.rows = n;
    b.x = adv(a.x, e0);
    b.y = per_row ? a.y : adv(a.y, e0);
    b.residual = adv(a.residual, e0);
    b.sum_out = adv(a.sum_out, e0);
    b.labels = adv(a.labels, r0);
    b.losses = adv(a.losses, r0);
    b.sums = adv(a.sums, r0);
    b.mins = adv(a.mins, r0);
    b.maxs = adv(a.maxs, r0);
    return b;
}

lr_status run(const Call& c, const lr_plan* forced, hipStream_t stream) {
    lr_status st = validate_call(c);
    if (st != LR_OK) return st;
    if (c.rows == 0) return LR_OK;  // nothing to launch
    const bool ce = c.op == LR_OP_CROSS_ENTROPY;
    const bool per_row = ce || c.op == LR_OP_ROW_SUM || c.op == LR_OP_ROW_MINMAX;
    const bool rows_aligned = c.cols % kVec == 0 && aligned16(c.x);
    const bool aligned = rows_aligned && (per_row || (aligned16(c.y) && aligned16(c.gamma) && aligned16(c.beta) &&
                                                      aligned16(c.residual) && aligned16(c.sum_out)));

    const bool have_ws = c.workspace != nullptr && c.workspace_bytes > 0;
    if (forced != nullptr && forced->family == LR_FAMILY_SPLIT &&
        (!have_ws || c.workspace_bytes < (uint64_t)plan_workspace_bytes(*forced, c.rows)))
        return LR_ERR_WORKSPACE;

    lr_device_facts facts;
    st = current_facts(&facts);
    if (st != LR_OK) return st;
    lr_plan plan;
    if (forced != nullptr) {
        st = validate_plan(&facts, c.op, c.rows, c.cols, c.policy, rows_aligned, forced);
        if (st != LR_OK) return st;
        plan = *forced;
    } else {
        // with a workspace large enough, the plan that may split rows;
        // otherwise the typed entry points' plan.  A norm called without
        // gamma and beta may have a plan of its own for that case.
        const bool params = c.gamma != nullptr || c.beta != nullptr;
        bool split_ok = false;
        if (have_ws) {
            lr_plan w;
            split_ok = plan_for_call(&facts, c.op, c.rows, c.cols, c.policy, rows_aligned, true, params, &w) ==
                           LR_OK &&
                       c.workspace_bytes >= (uint64_t)plan_workspace_bytes(w, c.rows);
            if (split_ok) plan = w;
        }
        if (!split_ok) {
            st = plan_for_call(&facts, c.op, c.rows, c.cols, c.policy, rows_aligned, false, params, &plan);
            if (st != LR_OK) return st;
        }
    }

    KArgs a;
    a.x = c.x;
    a.y = c.y;
    a.gamma = c.gamma;
    a.beta = c.beta;
    a.labels = c.labels;
    a.losses = c.losses;
    a.rows = c.rows;
    a.cols = (int32_t)c.cols;
    a.eps = c.eps;
    a.inv_cols = 1.0f / (float)c.cols;
    a.S = plan.waves_per_row;
    a.Q = plan.rows_per_block;
    a.team_magic = team_magic(plan.waves_per_row);
    auto same_phase = [&](const void* p) {
        return p == nullptr ? 1
                            : (int32_t)((reinterpret_cast<uintptr_t>(p) & 15u) ==
                                        (reinterpret_cast<uintptr_t>(c.x) & 15u));
    };
    a.y_same_phase = per_row ? 1 : same_phase(c.y);
    a.sums = c.sums;
    a.mins = c.mins;
    a.maxs = c.maxs;
    a.residual = c.residual;
    a.sum_out = c.sum_out;
    a.r_same_phase = same_phase(c.residual);
    a.s_same_phase = same_phase(c.sum_out);
    a.splits = plan.family == LR_FAMILY_SPLIT ? plan.splits : 0;
    a.ws = plan.family == LR_FAMILY_SPLIT ? static_cast<float*>(c.workspace) : nullptr;

    (void)hipGetLastError();  // clear a stale error so the launch's own status is seen
    // rows beyond one dispatch's reach run as consecutive pieces on `stream`
    const int64_t step = dispatch_rows(plan, c.rows);
    for (int64_t r0 = 0; r0 < c.rows; r0 += step) {
        const int64_t n = std::min(step, c.rows - r0);
        const hipError_t e = launch_piece(c.op, c.policy, piece_args(a, r0, n, per_row),
                                          piece_plan(plan, n), aligned, stream);
        if (e != hipSuccess) return LR_ERR_HIP;
    }
    return LR_OK;
}

}  // namespace
}  // namespace lr

using lr::Call;

extern "C" {

lr_status lr_softmax_f32(const float* x, float* y, int64_t rows, int64_t cols, lr_reduction_policy policy,
                         hipStream_t stream) {
    return lr::run(Call{LR_OP_SOFTMAX, x, nullptr, nullptr, y, nullptr, nullptr, rows, cols, 0.0f, policy},
                   nullptr, stream);
}

lr_status lr_rmsnorm_f32(const float* x, const float* gamma, float* y, int64_t rows, int64_t cols, float eps,
                         lr_reduction_policy policy, hipStream_t stream) {
    return lr::run(Call{LR_OP_RMSNORM, x, gamma, nullptr, y, nullptr, nullptr, rows, cols, eps, policy},
                   nullptr, stream);
}

lr_status lr_layernorm_f32(const float* x, const float* gamma, const float* beta, float* y, int64_t rows,
                           int64_t cols, float eps, lr_reduction_policy policy, hipStream_t stream) {
    return lr::run(Call{LR_OP_LAYERNORM, x, gamma, beta, y, nullptr, nullptr, rows, cols, eps, policy},
                   nullptr, stream);
}

lr_status lr_cross_entropy_f32(const float* logits, const int64_t* labels, float* losses, int64_t rows,
                               int64_t cols, lr_reduction_policy policy, hipStream_t stream) {
    return lr::run(
        Call{LR_OP_CROSS_ENTROPY, logits, nullptr, nullptr, nullptr, labels, losses, rows, cols, 0.0f, policy},
        nullptr, stream);
}

lr_status lr_add_layernorm_f32(const float* x, const float* residual, const float* gamma, const float* beta,
                               float* y, float* sum_out, int64_t rows, int64_t cols, float eps,
                               lr_reduction_policy policy, hipStream_t stream) {
    Call c{LR_OP_ADD_LAYERNORM, x, gamma, beta, y, nullptr, nullptr, rows, cols, eps, policy};
    c.residual = residual;
    c.sum_out = sum_out;
    return lr::run(c, nullptr, stream);
}

lr_status lr_row_sum_f32(const float* x, float* sums, int64_t rows, int64_t cols, lr_reduction_policy policy,
                         hipStream_t stream) {
    Call c{LR_OP_ROW_SUM, x, nullptr, nullptr, nullptr, nullptr, nullptr, rows, cols, 0.0f, policy};
    c.sums = sums;
    return lr::run(c, nullptr, stream);
}

lr_status lr_row_minmax_f32(const float* x, float* mins, float* maxs, int64_t rows, int64_t cols,
                            lr_reduction_policy policy, hipStream_t stream) {
    Call c{LR_OP_ROW_MINMAX, x, nullptr, nullptr, nullptr, nullptr, nullptr, rows, cols, 0.0f, policy};
    c.mins = mins;
    c.maxs = maxs;
    return lr::run(c, nullptr, stream);
}

static lr_status need_plan(const lr_plan* plan) { return plan == nullptr ? LR_ERR_NULL_POINTER : LR_OK; }

lr_status lr_copy_rows_f32(const float* x, float* y, int64_t rows, int64_t cols, const lr_plan* plan,
                           int32_t sync, hipStream_t stream) {
    if (plan == nullptr) return LR_ERR_NULL_POINTER;
    if (sync != 0 && sync != 1) return LR_ERR_INVALID_ARGUMENT;
    if (rows < 0 || cols <= 0 || rows > INT32_MAX || cols > INT32_MAX / 4) return LR_ERR_INVALID_SHAPE;
    if (rows == 0) return LR_OK;
    if (x == nullptr || y == nullptr) return LR_ERR_NULL_POINTER;
    if (cols % 4 != 0 || !lr::aligned16(x) || !lr::aligned16(y)) return LR_ERR_MISALIGNED;
    const int64_t tb = rows * cols * 4;
    if (x != y && lr::overlap(lr::range_of(x, tb), lr::range_of(y, tb))) return LR_ERR_ALIASING;
    const int S = plan->waves_per_row, n = plan->chunks_per_lane;
    const bool compiled = n == 1 || n == 2 || n == 3 || n == 4 || n == 6 || n == 8;
    if (plan->family != LR_FAMILY_CACHE || plan->rows_per_block != 1 || S < 1 || S > 16 ||
        plan->lanes_per_row != 64 * S || !compiled || (int64_t)64 * S * n * 4 < cols)
        return LR_ERR_UNREALIZABLE_PLAN;
    return lr::launch_copy_rows(x, y, rows, (int)cols, *plan, sync == 1, stream) == hipSuccess ? LR_OK : LR_ERR_HIP;
}

lr_status lr_softmax_f32_with_plan(const float* x, float* y, int64_t rows, int64_t cols,
                                   lr_reduction_policy policy, const lr_plan* plan, hipStream_t stream) {
    if (need_plan(plan) != LR_OK) return LR_ERR_NULL_POINTER;
    return lr::run(Call{LR_OP_SOFTMAX, x, nullptr, nullptr, y, nullptr, nullptr, rows, cols, 0.0f, policy},
                   plan, stream);
}

lr_status lr_rmsnorm_f32_with_plan(const float* x, const float* gamma, float* y, int64_t rows, int64_t cols,
                                   float eps, lr_reduction_policy policy, const lr_plan* plan,
                                   hipStream_t stream) {
    if (need_plan(plan) != LR_OK) return LR_ERR_NULL_POINTER;
    return lr::run(Call{LR_OP_RMSNORM, x, gamma, nullptr, y, nullptr, nullptr, rows, cols, eps, policy}, plan,
                   stream);
}

lr_status lr_layernorm_f32_with_plan(const float* x, const float* gamma, const float* beta, float* y,
                                     int64_t rows, int64_t cols, float eps, lr_reduction_policy policy,
                                     const lr_plan* plan, hipStream_t stream) {
    if (need_plan(plan) != LR_OK) return LR_ERR_NULL_POINTER;
    return lr::run(Call{LR_OP_LAYERNORM, x, gamma, beta, y, nullptr, nullptr, rows, cols, eps, policy}, plan,
                   stream);
}

lr_status lr_cross_entropy_f32_with_plan(const float* logits, const int64_t* labels, float* losses,
                                         int64_t rows, int64_t cols, lr_reduction_policy policy,
                                         const lr_plan* plan, hipStream_t stream) {
    if (need_plan(plan) != LR_OK) return LR_ERR_NULL_POINTER;
    return lr::run(
        Call{LR_OP_CROSS_ENTROPY, logits, nullptr, nullptr, nullptr, labels, losses, rows, cols, 0.0f, policy},
        plan, stream);
}

lr_status lr_add_layernorm_f32_with_plan(const float* x, const float* residual, const float* gamma,
                                         const float* beta, float* y, float* sum_out, int64_t rows,
                                         int64_t cols, float eps, lr_reduction_policy policy,
                                         const lr_plan* plan, hipStream_t stream) {
    if (need_plan(plan) != LR_OK) return LR_ERR_NULL_POINTER;
    Call c{LR_OP_ADD_LAYERNORM, x, gamma, beta, y, nullptr, nullptr, rows, cols, eps, policy};
    c.residual = residual;
    c.sum_out = sum_out;
    return lr::run(c, plan, stream);
}

lr_status lr_row_sum_f32_with_plan(const float* x, float* sums, int64_t rows, int64_t cols,
                                   lr_reduction_policy policy, const lr_plan* plan, hipStream_t stream) {
    if (need_plan(plan) != LR_OK) return LR_ERR_NULL_POINTER;
    Call c{LR_OP_ROW_SUM, x, nullptr, nullptr, nullptr, nullptr, nullptr, rows, cols, 0.0f, policy};
    c.sums = sums;
    return lr::run(c, plan, stream);
}

lr_status lr_row_minmax_f32_with_plan(const float* x, float* mins, float* maxs, int64_t rows, int64_t cols,
                                      lr_reduction_policy policy, const lr_plan* plan, hipStream_t stream) {
    if (need_plan(plan) != LR_OK) return LR_ERR_NULL_POINTER;
    Call c{LR_OP_ROW_MINMAX, x, nullptr, nullptr, nullptr, nullptr, nullptr, rows, cols, 0.0f, policy};
    c.mins = mins;
    c.maxs = maxs;
    return lr::run(c, plan, stream);
}

namespace {

// The call of lr_run_f32 (no workspace yet): members the operation does not
// use must be NULL.
lr_status run_call(lr_op op, const lr_tensors* t, int64_t rows, int64_t cols, float eps,
                   lr_reduction_policy policy, lr::Call* out) {
    if (t == nullptr) return LR_ERR_NULL_POINTER;
    if (op < LR_OP_SOFTMAX || op > LR_OP_ROW_MINMAX) return LR_ERR_INVALID_ARGUMENT;
    // members the operation does not use must be NULL
    const bool norm = op == LR_OP_RMSNORM || op == LR_OP_LAYERNORM || op == LR_OP_ADD_LAYERNORM;
    const bool ln = op == LR_OP_LAYERNORM || op == LR_OP_ADD_LAYERNORM;
    const bool dense_out = op == LR_OP_SOFTMAX || norm;
    if ((t->residual && op != LR_OP_ADD_LAYERNORM) || (t->gamma && !norm) || (t->beta && !ln) ||
        (t->labels && op != LR_OP_CROSS_ENTROPY) || (t->y && !dense_out) ||
        (t->sum_out && op != LR_OP_ADD_LAYERNORM) || (t->losses && op != LR_OP_CROSS_ENTROPY) ||
        (t->sums && op != LR_OP_ROW_SUM) || ((t->mins || t->maxs) && op != LR_OP_ROW_MINMAX))
        return LR_ERR_INVALID_ARGUMENT;
    Call c{op, t->x, t->gamma, t->beta, t->y, t->labels, t->losses, rows, cols, norm ? eps : 0.0f, policy};
    c.residual = t->residual;
    c.sum_out = t->sum_out;
    c.sums = t->sums;
    c.mins = t->mins;
    c.maxs = t->maxs;
    *out = c;
    return LR_OK;
}

}  // namespace

lr_status lr_run_f32(lr_op op, const lr_tensors* t, int64_t rows, int64_t cols, float eps,
                     lr_reduction_policy policy, const lr_plan* plan, void* workspace, uint64_t workspace_bytes,
                     hipStream_t stream) {
    Call c{};
    const lr_status st = run_call(op, t, rows, cols, eps, policy, &c);
    if (st != LR_OK) return st;
    c.workspace = workspace;
    c.workspace_bytes = workspace_bytes;
    return lr::run(c, plan, stream);
}

lr_status lr_run_f32_noalloc(lr_op op, const lr_tensors* t, int64_t rows, int64_t cols, float eps,
                             lr_reduction_policy policy, const lr_plan* plan, hipStream_t stream) {
    Call c{};
    lr_status st = run_call(op, t, rows, cols, eps, policy, &c);
    if (st != LR_OK) return st;
    // every argument is checked before the array's address is looked up
    st = lr::validate_call(c);
    if (st != LR_OK) return st;
    if (c.rows == 0) return LR_OK;
    if (plan != nullptr && lr_plan_workspace_bytes(plan, rows) > (uint64_t)LR_NOALLOC_SCRATCH_BYTES)
        return LR_ERR_WORKSPACE;
    void* ws = nullptr;
    st = lr::noalloc_scratch(&ws);
    if (st != LR_OK) return st;
    c.workspace = ws;
    c.workspace_bytes = LR_NOALLOC_SCRATCH_BYTES;
    return lr::run(c, plan, stream);
}

lr_status lr_workspace_query(lr_op op, int64_t rows, int64_t cols, lr_reduction_policy policy, uint64_t* bytes) {
    if (bytes == nullptr) return LR_ERR_NULL_POINTER;
    lr_device_facts f;
    lr_status st = lr::current_facts(&f);
    if (st != LR_OK) return st;
    // an aligned and a misaligned problem may plan differently: the larger need
    uint64_t need = 0;
    for (int32_t aligned = 0; aligned <= 1; ++aligned) {
        lr_plan p;
        st = lr_plan_for_device_ws(&f, op, rows, cols, policy, aligned, &p);
        if (st != LR_OK) return st;
        need = std::max(need, (uint64_t)lr::plan_workspace_bytes(p, rows));
    }
    *bytes = need;
    return LR_OK;
}

lr_status lr_device_facts_query(lr_device_facts* out) {
    if (out == nullptr) return LR_ERR_NULL_POINTER;
    return lr::current_facts(out);
}

lr_status lr_device_memory_query(int32_t* clock_khz, int32_t* bus_width_bits) {
    if (clock_khz == nullptr || bus_width_bits == nullptr) return LR_ERR_NULL_POINTER;
    int dev = 0, clk = 0, bus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&clk, hipDeviceAttributeMemoryClockRate, dev) != hipSuccess ||
        hipDeviceGetAttribute(&bus, hipDeviceAttributeMemoryBusWidth, dev) != hipSuccess)
        return LR_ERR_HIP;
    *clock_khz = clk;
    *bus_width_bits = bus;
    return LR_OK;
}

lr_status lr_plan_query(lr_op op, int64_t rows, int64_t cols, lr_reduction_policy policy, lr_plan* out) {
    if (out == nullptr) return LR_ERR_NULL_POINTER;
    lr_device_facts f;
    lr_status st = lr::current_facts(&f);
    if (st != LR_OK) return st;
    return lr_plan_for_device(&f, op, rows, cols, policy, 1, out);
}

const char* lr_status_string(lr_status s) {
    switch (s) {
        case LR_OK: return "LR_OK";
        case LR_ERR_NULL_POINTER: return "LR_ERR_NULL_POINTER: a required pointer is null";
        case LR_ERR_INVALID_SHAPE: return "LR_ERR_INVALID_SHAPE: rows/cols out of range";
        case LR_ERR_INVALID_EPS: return "LR_ERR_INVALID_EPS: eps must be finite and >= 0";
        case LR_ERR_INVALID_POLICY: return "LR_ERR_INVALID_POLICY: unknown reduction policy";
        case LR_ERR_MISALIGNED: return "LR_ERR_MISALIGNED: pointer not aligned to its element";
        case LR_ERR_ALIASING: return "LR_ERR_ALIASING: input and output ranges overlap";
        case LR_ERR_UNREALIZABLE_PLAN: return "LR_ERR_UNREALIZABLE_PLAN: plan cannot be realised as given";
        case LR_ERR_HIP: return "LR_ERR_HIP: the HIP runtime reported an error";
        case LR_ERR_INVALID_ARGUMENT: return "LR_ERR_INVALID_ARGUMENT: invalid argument";
        case LR_ERR_WORKSPACE: return "LR_ERR_WORKSPACE: the plan needs a larger workspace";
        default: return "unknown lr_status";
    }
}

const char* lr_version(void) { return "lr 0.1.0 gfx950"; }

}  // extern "C"
