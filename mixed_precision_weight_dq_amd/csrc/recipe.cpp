// Host side of bit allocation: the sensitivity of a matrix and the
// water-filling allocator that picks one bit width per matrix (the recipe).
//
// DynaQuant page (zingnex.cn): "第一步：敏感度测量" -- a matrix's sensitivity is
// its Hessian trace times the mean of its squared weights; "第二步：比特分配" --
// water-filling on a max-heap, each step raising one matrix by one level, the
// step with the most quality per byte first, in a hardware-native mode
// ({4, 8, 16}) or the full mode (4 .. 16), 16 meaning the BF16 weights are kept.
//
// Model of the predicted loss (the page gives the priority, not the loss): a
// matrix of sensitivity S kept at b < 16 bits loses S * 4^-b, at 16 bits
// nothing.  Uniform b-bit rounding leaves an error power proportional to the
// mean square weight times 4^-b, and the Hessian trace turns error power into
// loss, so this is the second-order loss up to one constant shared by all
// matrices.  A step from level a to level b removes S (4^-a - 4^-b) and adds
// params (b - a) / 8 bytes; its priority is the ratio.  Ties go to the lower
// matrix index; a step that does not fit in what is left of the budget is
// dropped (the budget only shrinks, so it never fits later) and the other
// matrices go on; a step that removes nothing is never taken.
//
// All arithmetic is fp64 in exactly the order written (no contraction), so the
// priorities, and therefore the chosen widths, are reproducible bit for bit.
#include "../../include/dq.h"

#include <algorithm>
#include <cmath>
#include <vector>

#pragma clang fp contract(off)

namespace {

struct Step {
    double priority;
    int64_t matrix;
};

// Heap order: the greater priority first, then the lower matrix index.
bool heap_less(const Step& a, const Step& b)
{
    if (a.priority != b.priority) return a.priority < b.priority;
    return a.matrix > b.matrix;
}

double step_priority(double s, int64_t params, int32_t b_from, int32_t b_to)
{
    const double lo = std::ldexp(1.0, -2 * b_from);
    const double hi = b_to >= DQ_TOP_BITS ? 0.0 : std::ldexp(1.0, -2 * b_to);
    const double gain = s * (lo - hi);
    const double nbytes = (double)(params * (int64_t)(b_to - b_from)) / 8.0;
    return gain / nbytes;
}

double level_loss(double s, int32_t bits)
{
    return bits >= DQ_TOP_BITS ? 0.0 : s * std::ldexp(1.0, -2 * bits);
}

}  // namespace

extern "C" {

dq_status dq_sensitivity(const double* h_trace, const double* sumsq, const int64_t* params,
                         int64_t n, double* out)
{
    if (!h_trace || !sumsq || !params || !out) return DQ_ERR_NULL;
    if (n < 1 || n > DQ_MAX_MATRICES) return DQ_ERR_SHAPE;
    for (int64_t i = 0; i < n; ++i) {
        if (!(std::isfinite(h_trace[i]) && h_trace[i] >= 0.0) ||
            !(std::isfinite(sumsq[i]) && sumsq[i] >= 0.0) || params[i] < 1 ||
            params[i] > DQ_MAX_PARAMS)
            return DQ_ERR_VALUE;
    }
    for (int64_t i = 0; i < n; ++i) {
        const double mean = sumsq[i] / (double)params[i];
        out[i] = h_trace[i] * mean;
    }
    return DQ_OK;
}

dq_status dq_allocate_bits(const double* sensitivity, const int64_t* params, int64_t n,
                           const int32_t* levels, int32_t n_levels, int64_t budget_bits,
                           int32_t* bits_out, int64_t* step_matrix, int32_t* step_bits,
                           int64_t step_capacity, int64_t* n_steps, double* loss)
{
    if (!sensitivity || !params || !levels || !bits_out) return DQ_ERR_NULL;
    if (step_capacity < 0) return DQ_ERR_SHAPE;
    if (step_capacity > 0 && (!step_matrix || !step_bits)) return DQ_ERR_NULL;
    if (n < 1 || n > DQ_MAX_MATRICES) return DQ_ERR_SHAPE;
    if (n_levels < 1 || n_levels > DQ_TOP_BITS - DQ_MIN_BITS + 1) return DQ_ERR_BITS;
    for (int32_t j = 0; j < n_levels; ++j) {
        if (levels[j] < DQ_MIN_BITS || levels[j] > DQ_TOP_BITS) return DQ_ERR_BITS;
        if (j > 0 && levels[j] <= levels[j - 1]) return DQ_ERR_BITS;
    }
    int64_t floor_bits = 0, top_bits = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (!(std::isfinite(sensitivity[i]) && sensitivity[i] >= 0.0) || params[i] < 1 ||
            params[i] > DQ_MAX_PARAMS)
            return DQ_ERR_VALUE;
        // up to 2^24 matrices of up to 2^40 parameters: the bit totals can
        // exceed int64 in the worst case, so they are checked
        if (__builtin_add_overflow(floor_bits, params[i] * levels[0], &floor_bits) ||
            __builtin_add_overflow(top_bits, params[i] * levels[n_levels - 1], &top_bits))
            return DQ_ERR_VALUE;
    }
    const int64_t budget = budget_bits < 0 ? top_bits : budget_bits;
    if (budget < floor_bits) return DQ_ERR_BUDGET;

    std::vector<int32_t> lvl((size_t)n, 0);
    std::vector<Step> heap;
    heap.reserve((size_t)n);
    if (n_levels > 1) {
        for (int64_t i = 0; i < n; ++i) {
            const double p = step_priority(sensitivity[i], params[i], levels[0], levels[1]);
            if (p > 0.0) heap.push_back({p, i});
        }
        std::make_heap(heap.begin(), heap.end(), heap_less);
    }
    int64_t used = floor_bits, steps = 0;
    while (!heap.empty()) {
        std::pop_heap(heap.begin(), heap.end(), heap_less);
        const Step top = heap.back();
        heap.pop_back();
        const int64_t i = top.matrix;
        const int32_t j = lvl[(size_t)i];
        const int64_t cost = params[i] * (int64_t)(levels[j + 1] - levels[j]);
        if (used + cost > budget) continue;  // dropped for good
        used += cost;
        lvl[(size_t)i] = j + 1;
        if (steps < step_capacity) {
            step_matrix[steps] = i;
            step_bits[steps] = levels[j + 1];
        }
        ++steps;
        if (j + 2 < n_levels) {
            const double p = step_priority(sensitivity[i], params[i], levels[j + 1], levels[j + 2]);
            if (p > 0.0) {
                heap.push_back({p, i});
                std::push_heap(heap.begin(), heap.end(), heap_less);
            }
        }
    }
    double total = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        bits_out[i] = levels[lvl[(size_t)i]];
        total += level_loss(sensitivity[i], bits_out[i]);
    }
    if (n_steps) *n_steps = steps;
    if (loss) *loss = total;
    return DQ_OK;
}

}  // extern "C"
