// Host-side accuracy check of the library's fp64 exp for y <= 0 (built with
// hipcc, runs on the CPU): prints the largest relative error against exp().
#include <cmath>
#include <cstdio>
#include <random>

#include "tv_device.h"

int main() {
    double tab[32];
    for (int j = 0; j < 32; ++j) tv::exp2_table(tab, j);
    std::mt19937_64 g(12345);
    std::uniform_real_distribution<double> wide(-745.0, 0.0), narrow(-40.0, 0.0), tiny(-1e-6, 0.0);
    double worst = 0.0, worst_y = 0.0;
    for (int i = 0; i < 3000000; ++i) {
        const double y = i % 3 == 0 ? wide(g) : (i % 3 == 1 ? narrow(g) : tiny(g));
        const double ref = std::exp(y);
        if (ref < 1e-300) continue;  // subnormal range: absolute error only
        const double err = std::fabs(tv::exp_nonpos(y, tab) - ref) / ref;
        if (err > worst) { worst = err; worst_y = y; }
    }
    const double edge[] = {0.0, -0.0, -1e-300, -0.010830424696249145, -0.6931471805599453, -700.0, -745.0, -746.0};
    for (double y : edge) {
        const double ref = std::exp(y), got = tv::exp_nonpos(y, tab);
        const double err = ref > 1e-300 ? std::fabs(got - ref) / ref : std::fabs(got - ref);
        if (err > worst) { worst = err; worst_y = y; }
    }
    std::printf("%.3e %.17g\n", worst, worst_y);
    return 0;
}
