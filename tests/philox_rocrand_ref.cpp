// Test helper: prints rocRAND's Philox-4x32-10 engine output for given
// (seed, node, seq, purpose) lines on stdin.  Host-only; no GPU is touched.
// rocRAND's state counter is (offset/4 lo, offset/4 hi, subsequence lo,
// subsequence hi), so counter (node, seq, purpose, 0) is reached with
// subsequence = purpose and offset = 4 * ((seq << 32) | node), seq < 2^30.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
int main() {
    unsigned long long seed;
    unsigned node, seq, purpose;
    while (std::scanf("%llu %u %u %u", &seed, &node, &seq, &purpose) == 4) {
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, purpose, 4ULL * (((unsigned long long)seq << 32) | node), &st);
        uint4 r = rocrand4(&st);
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
