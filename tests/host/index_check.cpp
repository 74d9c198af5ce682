// Host-only check of the pass geometry's index logic: exact multiply-shift
// division against plain division, the (window, slot) -> token map being a
// bijection onto the grid that agrees with the coordinate definition, and on
// padded grids the packed coordinates, mirror images and side-buffer indices.
#include "squad_internal.h"

#include <cstdio>
#include <cstdlib>
#include <vector>

using namespace squad;

static int failures = 0;

static void check_div(uint32_t d) {
    const FastDiv f = make_fastdiv(d);
    uint64_t x = 88172645463325252ull;
    for (int i = 0; i < 20000; ++i) {
        x ^= x << 13; x ^= x >> 7; x ^= x << 17;
        const uint32_t n = (uint32_t)(x & 0x7fffffffu);
        if (fdiv(n, f) != n / d) { if (failures++ < 10) std::printf("div %u / %u\n", n, d); }
    }
    const uint32_t edges[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 0x7fffffffu, 0x7ffffffeu, 0x40000000u};
    for (uint32_t n : edges)
        if (n <= 0x7fffffffu && fdiv(n, f) != n / d) { if (failures++ < 10) std::printf("div %u / %u\n", n, d); }
}

static void check_geometry(int T, int Hs, int Ws, int wt, int wh, int ww) {
    PassGeom g{};
    g.n = (int64_t)T * Hs * Ws;
    g.Hs = Hs; g.Ws = Ws; g.wt = wt; g.wh = wh; g.ww = ww;
    g.Cy = Hs / wh; g.Cx = Ws / ww;
    g.div_wins_t = make_fastdiv((uint32_t)(g.Cy * g.Cx));
    g.div_Cx = make_fastdiv((uint32_t)g.Cx);
    g.div_slots_t = make_fastdiv((uint32_t)(wh * ww));
    g.div_ww = make_fastdiv((uint32_t)ww);
    const int m = wt * wh * ww, nw = (int)(g.n / m);
    std::vector<int> seen(g.n, 0);
    for (int c = 0; c < nw; ++c)
        for (int j = 0; j < m; ++j) {
            const int i = win_origin(g, c) + slot_offset(g, j);
            if (i < 0 || i >= g.n) { if (failures++ < 10) std::printf("token out of range\n"); continue; }
            ++seen[i];
            const int t = i / (Hs * Ws), y = (i / Ws) % Hs, x = i % Ws;
            const int cw = ((t / wt) * g.Cy + y / wh) * g.Cx + x / ww;
            const int js = ((t % wt) * wh + y % wh) * ww + x % ww;
            if (cw != c || js != j) { if (failures++ < 10) std::printf("map mismatch c=%d j=%d\n", c, j); }
        }
    for (int64_t i = 0; i < g.n; ++i)
        if (seen[i] != 1) { if (failures++ < 10) std::printf("token %lld seen %d times\n", (long long)i, seen[i]); }
}

static void check_decode(int B, int heads, int P) {
    PassGeom g{};
    g.heads = heads; g.P = P;
    g.div_heads = make_fastdiv((uint32_t)heads);
    g.div_P = make_fastdiv((uint32_t)P);
    for (int p = 0; p < B * heads * P; ++p) {
        const ProblemIndex pr = decode_problem(g, p);
        if (pr.h != p % heads || pr.pi != (p / heads) % P || pr.b != p / (heads * P)) {
            if (failures++ < 10) std::printf("decode %d\n", p);
        }
    }
}

// Padded grid (T, Hp, Wp) over the real (T, Hs, Ws): (window, slot) covers
// every padded position once through packed coordinates; real positions name
// their own token, padded ones the mirror image about the last row / column;
// side-buffer indices enumerate the padded positions exactly once.
static void check_padded(int T, int Hs, int Ws, int wt, int wh, int ww) {
    const int Hp = (Hs + wh - 1) / wh * wh, Wp = (Ws + ww - 1) / ww * ww;
    PassGeom g{};
    g.n = (int64_t)T * Hs * Ws;
    g.Hs = Hs; g.Ws = Ws; g.wt = wt; g.wh = wh; g.ww = ww;
    g.Cy = Hp / wh; g.Cx = Wp / ww;
    g.pad = 1; g.Hp = Hp; g.Wp = Wp;
    g.pad_per_frame = Hs * (Wp - Ws) + (Hp - Hs) * Wp;
    g.npad = (int64_t)T * g.pad_per_frame;
    g.div_wins_t = make_fastdiv((uint32_t)(g.Cy * g.Cx));
    g.div_Cx = make_fastdiv((uint32_t)g.Cx);
    g.div_slots_t = make_fastdiv((uint32_t)(wh * ww));
    g.div_ww = make_fastdiv((uint32_t)ww);
    const int m = wt * wh * ww, nw = T * Hp * Wp / m;
    std::vector<int> seen((size_t)T * Hp * Wp, 0), pad_seen((size_t)g.npad, 0);
    for (int c = 0; c < nw; ++c)
        for (int j = 0; j < m; ++j) {
            const int p = win_coords(g, c) + slot_coords(g, j);
            const int t = p >> 20, y = (p >> 10) & 1023, x = p & 1023;
            // the same position from the plain definition of window and slot
            const int ct = c / (g.Cy * g.Cx), cy = (c / g.Cx) % g.Cy, cx = c % g.Cx;
            const int jt = j / (wh * ww), jy = (j / ww) % wh, jx = j % ww;
            if (t != ct * wt + jt || y != cy * wh + jy || x != cx * ww + jx) {
                if (failures++ < 10) std::printf("padded coords c=%d j=%d\n", c, j);
                continue;
            }
            ++seen[((size_t)t * Hp + y) * Wp + x];
            const int ys = y < Hs ? y : Hs - 1 - (y - (Hs - 1));
            const int xs = x < Ws ? x : Ws - 1 - (x - (Ws - 1));
            if (ys < 0 || xs < 0 || mirrored_token(g, p) != (t * Hs + ys) * Ws + xs) {
                if (failures++ < 10) std::printf("mirror c=%d j=%d\n", c, j);
            }
            const bool real = y < Hs && x < Ws;
            if (is_real(g, p) != real) { if (failures++ < 10) std::printf("is_real c=%d j=%d\n", c, j); }
            if (!real) {
                const int k = pad_index(g, p);
                if (k < 0 || k >= g.npad) { if (failures++ < 10) std::printf("pad index range\n"); continue; }
                ++pad_seen[k];
            }
        }
    for (size_t i = 0; i < seen.size(); ++i)
        if (seen[i] != 1) { if (failures++ < 10) std::printf("padded position %zu seen %d times\n", i, seen[i]); }
    for (size_t i = 0; i < pad_seen.size(); ++i)
        if (pad_seen[i] != 1) { if (failures++ < 10) std::printf("pad index %zu seen %d times\n", i, pad_seen[i]); }
}

int main() {
    for (uint32_t d = 1; d < 3000; ++d) check_div(d);
    const uint32_t big[] = {65535u, 65536u, 65537u, 1000003u, 0x3fffffffu, 0x40000000u, 0x40000001u, 0x7fffffffu};
    for (uint32_t d : big) check_div(d);
    check_geometry(21, 22, 40, 21, 2, 4);
    check_geometry(21, 30, 52, 21, 2, 4);
    check_geometry(21, 44, 80, 21, 4, 4);
    check_geometry(3, 4, 4, 3, 2, 2);
    check_geometry(2, 9, 34, 1, 1, 17);
    check_geometry(8, 8, 8, 1, 1, 1);
    check_geometry(8, 8, 8, 8, 8, 8);
    check_geometry(4, 6, 10, 2, 3, 5);
    check_padded(21, 22, 40, 21, 2, 3);
    check_padded(2, 5, 7, 2, 3, 2);
    check_padded(3, 7, 13, 1, 4, 5);
    check_padded(1, 9, 2, 1, 9, 2);
    check_padded(21, 45, 80, 21, 4, 3);
    check_padded(4, 6, 6, 2, 6, 6);
    check_padded(5, 1, 11, 5, 1, 4);
    check_decode(2, 40, 220);
    check_decode(1, 24, 168);
    check_decode(3, 1, 7);
    if (failures) { std::printf("FAILED: %d\n", failures); return 1; }
    std::printf("OK\n");
    return 0;
}
