// Host check of lr::wave_elems (row_reductions_amd/csrc/lr_map.hpp), the
// count of a row's elements that one wavefront of a whole-wave team holds:
// for every team size S, every compiled chunk count, every phase and a
// spread of row lengths the team covers, it must equal a brute-force count
// over the wave's lanes and chunk slots built from the same chunk_index /
// elem_index / elem_valid functions the kernels use, and the waves' counts
// must add up to the row length.
#include <cstdio>
#include <cstdlib>

#include "lr_map.hpp"

using namespace lr;

static int brute(int s, int W, int nch, int phase, int cols) {
    int n = 0;
    for (int lane = 0; lane < kWave; ++lane)
        for (int c = 0; c < nch; ++c) {
            const int k = chunk_index(s * kWave + lane, W, c);
            for (int j = 0; j < kVec; ++j) n += elem_valid(elem_index(k, j, phase), cols) ? 1 : 0;
        }
    return n;
}

int main() {
    const int nchs[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32};
    long checked = 0;
    unsigned seed = 12345u;
    for (int S = 1; S <= 16; ++S)
        for (int nch : nchs)
            for (int phase = 0; phase < kVec; ++phase) {
                const int W = kWave * S;
                const int cap = kVec * W * nch - phase;  // the longest row the team covers
                int lens[40];
                int m = 0;
                for (int c = 1; c <= 8 && c <= cap; ++c) lens[m++] = c;
                for (int d = 0; d < 8; ++d) lens[m++] = cap - d > 0 ? cap - d : 1;
                for (int d = 0; d < 24; ++d) {
                    seed = seed * 1103515245u + 12345u;
                    lens[m++] = 1 + (int)((seed >> 8) % (unsigned)cap);
                }
                for (int i = 0; i < m; ++i) {
                    const int cols = lens[i];
                    int total = 0;
                    for (int s = 0; s < S; ++s) {
                        const int a = wave_elems(s, W, nch, phase, cols);
                        const int b = brute(s, W, nch, phase, cols);
                        if (a != b) {
                            std::printf("MISMATCH S=%d nch=%d phase=%d cols=%d wave %d: %d vs %d\n", S, nch, phase,
                                        cols, s, a, b);
                            return 1;
                        }
                        total += a;
                        ++checked;
                    }
                    if (total != cols) {
                        std::printf("SUM S=%d nch=%d phase=%d cols=%d: %d\n", S, nch, phase, cols, total);
                        return 1;
                    }
                }
            }
    std::printf("%ld wave counts checked\n", checked);
    return 0;
}
