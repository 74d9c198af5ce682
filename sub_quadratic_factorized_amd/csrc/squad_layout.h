// LDS block layouts of the bf16 pass kernel, as host+device functions so that
// a host-only check can verify every address (alignment, bounds, and that each
// fetch returns the element the MFMA operand expects).
#pragma once

#include <hip/hip_runtime.h>

namespace squad {

constexpr int kBlockRows = 32;  // rows per streamed block

template <int D>
struct BlockGeo {
    static constexpr int KC = D / 8;              // 16-byte chunks per row
    static constexpr int NCH = kBlockRows * KC;   // chunks per block
    static constexpr int KS = D / 32;             // k-steps of the score MFMA
    static constexpr int DT = D / 16;             // 16-row d tiles of the output
    // K and Q rows padded by 32 B: operand fetches (16 rows, one 16-byte column
    // each) are free of bank conflicts at this stride on gfx950 (measured).
    static constexpr int KSTR = D + 16;
    // V rows are not padded; instead 16-byte column c of row r sits at column
    // c ^ 4*(r mod QW) with its two 8-byte halves swapped when bit log2(QW) of
    // r is set (QW = KC/4).  Each 32-lane half of a transposing fetch (8 rows x
    // 4 pieces of 8 bytes) then covers every bank exactly once (measured).
    static constexpr int VSTR = D;
    static constexpr int QW = KC / 4;
};

// Element offset, inside a V block, of the 16-byte column c of row r (where
// the whole 16-byte chunk is stored; 16-byte aligned).
template <int D>
__host__ __device__ inline int v_chunk_offset(int r, int c) {
    using G = BlockGeo<D>;
    return r * G::VSTR + (c ^ (4 * (r & (G::QW - 1)))) * 8;
}

// Whether row r stores its 8-byte halves swapped.
template <int D>
__host__ __device__ inline bool v_halves_swapped(int r) {
    return ((r / BlockGeo<D>::QW) & 1) != 0;
}

// Element offset of half h (elements 4h..4h+3) of logical 16-byte column c of
// row r (8-byte aligned): what a transposing fetch addresses.
template <int D>
__host__ __device__ inline int v_half_offset(int r, int c, int h) {
    return v_chunk_offset<D>(r, c) + 4 * (h ^ (v_halves_swapped<D>(r) ? 1 : 0));
}

// d index held by row r of output d-tile dt.  Tiles are used in pairs so that
// a lane's 4+4 accumulator rows cover 8 consecutive d (one 16-byte store).
__host__ __device__ inline int dmap(int dt, int r) {
    return 32 * (dt >> 1) + 8 * (r >> 2) + 4 * (dt & 1) + (r & 3);
}

// Row of a V block that lane (li, lg) addresses in its transposing fetch
// (the low 16 keys; the high fetch uses this row + 16), and the logical
// 16-byte column / half for d-tile dt.
__host__ __device__ inline int v_fetch_row(int li, int lg) { return 4 * lg + (li >> 2); }
__host__ __device__ inline int v_fetch_col(int li, int dt) { return 4 * (dt >> 1) + (li & 3); }
__host__ __device__ inline int v_fetch_half(int dt) { return dt & 1; }

}  // namespace squad
