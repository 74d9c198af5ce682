// Host-only check of the bf16 pass kernel's LDS block layouts (no GPU used):
// every store/fetch address is aligned and in bounds, the staged chunks of a
// block tile it exactly once, and every fetch returns the element the MFMA
// operand layout expects (the transposing fetch emulated from its measured
// lane semantics: output lane i of a 16-lane group gets, as element t, element
// i%4 of the 8 bytes addressed by lane 4t + i/4 of the same group).
#include "squad_layout.h"

#include <cstdio>
#include <vector>

using namespace squad;

static int failures = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            if (failures < 20) std::printf(__VA_ARGS__); \
            ++failures;                                   \
        }                                                 \
    } while (0)

template <int D>
void check_v() {
    using G = BlockGeo<D>;
    const int size = kBlockRows * G::VSTR;
    std::vector<long> v(size, -1);
    // stores: chunk ch = (row, 16-byte column); on swapped row groups its two
    // 8-byte halves trade places (the kernels store each half at its own address)
    for (int ch = 0; ch < G::NCH; ++ch) {
        const int r = ch / G::KC, c = ch % G::KC;
        const int base = v_chunk_offset<D>(r, c);
        CHECK(base % 8 == 0, "D=%d V store row %d col %d misaligned (%d)\n", D, r, c, base);
        CHECK(base >= 0 && base + 8 <= size, "D=%d V store row %d col %d out of bounds\n", D, r, c);
        if (base < 0 || base + 8 > size) continue;
        for (int e = 0; e < 8; ++e) {
            const int le = v_halves_swapped<D>(r) ? (e + 4) % 8 : e;  // logical element at physical e
            CHECK(v[base + e] == -1, "D=%d V element written twice at %d\n", D, base + e);
            v[base + e] = (long)r * D + 8 * c + le;
        }
    }
    for (int i = 0; i < size; ++i) CHECK(v[i] != -1, "D=%d V element %d never written\n", D, i);
    // transposing fetches
    for (int part = 0; part < 2; ++part)
        for (int dt = 0; dt < G::DT; ++dt)
            for (int lg = 0; lg < 4; ++lg) {
                long piece[16][4];
                for (int j = 0; j < 16; ++j) {
                    const int row = v_fetch_row(j, lg) + 16 * part;
                    const int off = v_half_offset<D>(row, v_fetch_col(j, dt), v_fetch_half(dt));
                    CHECK(off % 4 == 0 && off >= 0 && off + 4 <= size, "D=%d V fetch misaligned/out of bounds\n", D);
                    for (int e = 0; e < 4; ++e) piece[j][e] = (off >= 0 && off + 4 <= size) ? v[off + e] : -2;
                }
                for (int i = 0; i < 16; ++i)
                    for (int t = 0; t < 4; ++t) {
                        const long got = piece[4 * t + i / 4][i % 4];
                        const long key = 4 * lg + t + 16 * part;
                        const long want = key * D + dmap(dt, i);
                        CHECK(got == want, "D=%d V fetch dt=%d lg=%d lane=%d t=%d part=%d: got %ld want %ld\n", D, dt,
                              lg, i, t, part, got, want);
                    }
            }
}

template <int D>
void check_k_and_q(int lmax) {
    using G = BlockGeo<D>;
    const int size = kBlockRows * G::KSTR;
    std::vector<long> k(size, -1);
    for (int ch = 0; ch < G::NCH; ++ch) {
        const int r = ch / G::KC, col = (ch % G::KC) * 8;
        const int off = r * G::KSTR + col;
        CHECK(off % 8 == 0 && off + 8 <= size, "D=%d K store misaligned/out of bounds\n", D);
        for (int e = 0; e < 8; ++e) k[off + e] = (long)r * D + col + e;
    }
    // score-operand fetch: lane (li, lg), k-step s, half h2: row 16*h2 + li, 16-byte column 4s + lg
    for (int h2 = 0; h2 < 2; ++h2)
        for (int s = 0; s < G::KS; ++s)
            for (int lg = 0; lg < 4; ++lg)
                for (int li = 0; li < 16; ++li) {
                    const int off = (16 * h2 + li) * G::KSTR + (4 * s + lg) * 8;
                    CHECK(off % 8 == 0 && off + 8 <= size, "D=%d K fetch misaligned/out of bounds\n", D);
                    for (int e = 0; e < 8; ++e)
                        CHECK(k[off + e] == (long)(16 * h2 + li) * D + (4 * s + lg) * 8 + e, "D=%d K fetch value\n",
                              D);
                }
    // Q stage: rows up to the padded longest problem
    const int qrows = (lmax + kBlockRows - 1) / kBlockRows * kBlockRows;
    const int nb = (lmax + kBlockRows - 1) / kBlockRows;
    for (int blk = 0; blk < nb; ++blk)
        for (int ch = 0; ch < G::NCH; ++ch) {
            const int off = (blk * kBlockRows + ch / G::KC) * G::KSTR + (ch % G::KC) * 8;
            CHECK(off % 8 == 0 && off + 8 <= qrows * G::KSTR, "D=%d Q store out of bounds (lmax %d)\n", D, lmax);
        }
}

int main() {
    check_v<128>();
    check_v<64>();
    for (int lmax : {192, 256, 384}) {
        check_k_and_q<128>(lmax);
        check_k_and_q<64>(lmax);
    }
    if (failures) {
        std::printf("FAILED: %d problems\n", failures);
        return 1;
    }
    std::printf("OK\n");
    return 0;
}
