// Host-side planning of the dense product's split tail, kept apart from the
// kernels so that the host logic can also be built and checked on its own.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstdint>

namespace mx {

constexpr int64_t PLAN_BM = 256, PLAN_BN = 256, PLAN_BK = 128;  // output tile; K per cost unit

// With T tiles on P compute units the last R = T mod P tiles form a partial
// round that leaves most units idle.  Each of them is cut into S K ranges (at
// most P / R, at most one per 256-K group), one workgroup per range: the round
// then costs about 1/S of a tile, plus writing and summing R * S partial tiles
// of 256 KiB.  A tile costs ~1.7 us per 128-K stage and summing one partial
// ~0.065 us, so S ~ sqrt(26 * stages / R) balances the two.  Only BF16 C
// stored by whole-line stores (every tile full width) is split.  S depends on
// the shape and the compute-unit count only, so the summation order (and the
// bytes of C) is fixed per shape and device.
struct SplitPlan {
    int64_t rem = 0, S = 0;
    int64_t bytes() const { return S >= 2 ? rem * S * PLAN_BM * PLAN_BN * 4 : 0; }
};

inline SplitPlan split_plan(int64_t M, int64_t N, int64_t K, int c_dtype, bool vec16, int64_t cus)
{
    SplitPlan sp;
    if (M <= 0 || N <= 0 || K <= 0 || cus <= 0)
        return sp;
    const int64_t tiles = ((M + PLAN_BM - 1) / PLAN_BM) * ((N + PLAN_BN - 1) / PLAN_BN);
    const int64_t groups = (K / PLAN_BK + 1) / 2;
    const int64_t rem = tiles % cus;
    if (rem > 0 && groups >= 2 && c_dtype == 0 && vec16 && N % PLAN_BN == 0) {
        const int64_t balance = std::max<int64_t>(2, (int64_t)std::sqrt(26.0 * 2 * groups / (double)rem));
        sp.S = std::min<int64_t>(std::min<int64_t>(cus / rem, groups), balance);
        sp.rem = rem;
    }
    return sp;
}

}  // namespace mx
