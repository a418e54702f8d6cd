// fastdiv.h -- division by a launch constant: the host side of the kernels'
// index arithmetic (internal to the library; no HIP dependency).
#pragma once

#include <cstdint>

namespace dgw {

// Division by a launch constant d (1 <= d <= 2^31) of an index n in
// [0, 2^31) without a divide sequence: with s = ceil(log2 d) and
// m = ceil(2^(32+s) / d) (so 2^32 <= m < 2^33), floor(n / d) =
// floor(n m / 2^(32+s)) = (umulhi(n, m - 2^32) + n) >> s.  Exact: the error
// of m, m d - 2^(32+s), is below d <= 2^s, so n m / 2^(32+s) exceeds n / d by
// less than n / 2^(32+s) < 1 / (2 d), which cannot reach the next integer.
// The kernels evaluate the last form in 32-bit arithmetic (umulhi(n, m') < n,
// so the sum stays below 2^32).
struct FastDiv {
    uint32_t m;   // m - 2^32
    uint32_t s;
};

// The constants of d; d < 1 gives those of 1 (a divisor the launch does not use).
inline FastDiv fast_div(int64_t d) {
    if (d < 1) d = 1;
    uint32_t s = 0;
    while ((int64_t(1) << s) < d) ++s;
    const uint64_t m = ((uint64_t(1) << (32 + s)) + uint64_t(d) - 1) / uint64_t(d);   // in [2^32, 2^33)
    return FastDiv{uint32_t(m - (uint64_t(1) << 32)), s};
}

}  // namespace dgw
