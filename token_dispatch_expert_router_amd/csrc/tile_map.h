// Tile maps of the grouped GEMM (gemm_mfma.hip): which output tile a block computes,
// and how many blocks a pass launches.  Compiled into the kernels and, unchanged, into a
// host program that walks every block of a launch over given segment offsets and checks
// that each output tile is produced exactly once and inside its segment.
//
// The experts' rows are contiguous segments [offsets[e], offsets[e+1]) of the permuted
// buffer whose sizes live only in device memory, so a block of a row-segmented pass
// finds its (expert, m-tile, n-tile) from `offsets` itself.  Blocks are dispatched
// round-robin over the 8 XCDs (block b runs on XCD b & 7); the maps give each XCD
// contiguous runs of tiles, in which consecutive tiles form 4 x N blocks (groups of four
// m-tiles, M fastest) whose operand panels stay in that XCD's L2.
#pragma once

#include "common.h"

namespace moe {
namespace tiles {

constexpr int BM = 256;  // output rows per tile
constexpr int BN = 256;  // output columns per tile (the gate/up forward: 128 of W_g + 128 of W_u)
constexpr int GROUP_M = 4;
constexpr int NXCD = 8;

// Row tiles over all segments.
__host__ __device__ __forceinline__ int count_row_tiles(const int32_t* offsets, int E) {
    int mt = 0;
    for (int i = 0; i < E; ++i) mt += (offsets[i + 1] - offsets[i] + BM - 1) / BM;
    return mt;
}

// Logical tile L of `valid` goes to XCD L / ceil(valid / 8), so that each XCD runs a
// contiguous range of equal length; returns -1 for a block with no tile.
__host__ __device__ __forceinline__ int xcd_remap(int b, int valid) {
    const int per = (valid + NXCD - 1) / NXCD;
    const int j = b / NXCD;
    if (j >= per) return -1;
    const int L = (b % NXCD) * per + j;
    return L < valid ? L : -1;
}

// Tiles of one segment (or one expert's weight gradient) are ordered in groups of
// GROUP_M m-tiles, m fastest inside a group, so the ~32 consecutive tiles one XCD runs
// at a time form a 4 x 8 block that shares 4 row panels and 8 weight panels, however
// many m-tiles the segment has.
__host__ __device__ __forceinline__ void grouped_mn(int loc, int mt, int n_tiles, int& mi,
                                                    int& ni) {
    const int gi = loc / (GROUP_M * n_tiles);
    const int rest = mt - gi * GROUP_M;
    const int gm = rest < GROUP_M ? rest : GROUP_M;
    const int idx = loc - gi * GROUP_M * n_tiles;
    mi = gi * GROUP_M + idx % gm;
    ni = idx / gm;
}

// (first row, tile height) of m-tile mi of a segment [lo, hi).  With `half`, a segment's
// last row tile is 128 rows high when it holds at most 128 rows (the tile count does not
// change); every other tile is BM rows high.
__host__ __device__ __forceinline__ void row_extent(int lo, int hi, int mi, bool half, int& m0,
                                                    int& mh) {
    m0 = lo + mi * BM;
    mh = (half && hi - m0 <= BM / 2) ? BM / 2 : BM;
}

// The row maps (which XCD runs which tile of a row pass), chosen per launch (row_map).
enum RowMap { ROW_CONTIGUOUS = 0, ROW_SHARED = 1, ROW_CHUNKED = 2 };
constexpr int CHUNK = 32;  // tiles per chunk of the chunked map: one XCD's tiles in flight

// Row passes: (expert, first row, segment end, n-tile, tile height) of block b, false
// for a block with no tile.  Block b runs the (b / 8)-th tile of XCD b % 8's sequence
// under one of three maps of the logical tile order (the segments in order, each
// segment's tiles in grouped order):
//  - contiguous: the order is cut into eight equal contiguous ranges, one per XCD, so an
//    XCD keeps its experts' row panels to itself;
//  - chunked: the order is cut into chunks of CHUNK tiles dealt round-robin to the XCDs,
//    so an XCD still runs 4 x 8 blocks while the eight XCDs run eight neighbouring
//    chunks, the same expert's rows and adjacent weight columns, at the same time;
//  - shared: XCD x takes the same contiguous eighth of every segment's tile order, tiles
//    [x T / 8, (x + 1) T / 8) of a segment of T tiles, segment after segment, so all XCDs
//    work on the same experts at the same time (weight columns that several XCDs need
//    for different row groups are fetched from HBM once and served to the others by the
//    last-level cache) and each streams the same share of every expert's weights,
//    however unequal the segments.
__host__ __device__ __forceinline__ bool row_tile(int b, const int32_t* offsets, int E,
                                                  int n_tiles, bool half, int map, int& e,
                                                  int& m0, int& m_lim, int& nt, int& mh) {
    int mi;
    const int x = b % NXCD;
    const int j = b / NXCD;
    if (map != ROW_SHARED) {
        const int valid = count_row_tiles(offsets, E) * n_tiles;
        int L;
        if (map == ROW_CHUNKED) {
            L = ((j / CHUNK) * NXCD + x) * CHUNK + j % CHUNK;
            if (L >= valid) return false;
        } else {
            L = xcd_remap(b, valid);
            if (L < 0) return false;
        }
        int acc = 0;
        for (int i = 0; i < E; ++i) {
            const int lo = offsets[i], hi = offsets[i + 1];
            const int mt = (hi - lo + BM - 1) / BM;
            const int tiles = mt * n_tiles;
            if (L < acc + tiles) {
                grouped_mn(L - acc, mt, n_tiles, mi, nt);
                e = i;
                m_lim = hi;
                row_extent(lo, hi, mi, half, m0, mh);
                return true;
            }
            acc += tiles;
        }
        return false;
    }
    int acc = 0;
    for (int i = 0; i < E; ++i) {
        const int lo = offsets[i], hi = offsets[i + 1];
        const int mt = (hi - lo + BM - 1) / BM;
        const unsigned tiles = (unsigned)(mt * n_tiles);
        const int t0 = (int)((uint64_t)x * tiles / NXCD);
        const int cnt = (int)((uint64_t)(x + 1) * tiles / NXCD) - t0;
        if (j < acc + cnt) {
            grouped_mn(t0 + (j - acc), mt, n_tiles, mi, nt);
            e = i;
            m_lim = hi;
            row_extent(lo, hi, mi, half, m0, mh);
            return true;
        }
        acc += cnt;
    }
    return false;
}

// Which row map a launch takes, by measurement on the layer shapes (R rows of buffer
// bound over E experts; kernel traces, the three maps in turn on one MI355X):
//  - more than 1024 rows per expert (two or more groups of four m-tiles): shared on every
//    row pass (4-8% faster than contiguous, 1-3% faster than chunked);
//  - 641-1024 rows (one group of four m-tiles): chunked for the forward passes (3% faster
//    than contiguous; shared makes the down forward 5% slower) and shared for the dgrads
//    (3-4% faster than contiguous, the gate/up dgrad 3% faster than chunked);
//  - at most 640 rows (one or two m-tiles per expert, whose row panels the shared and
//    chunked maps send to several XCDs): shared for the gate/up forward, whose
//    half-height last tiles otherwise leave the XCDs unequal work (6% faster), and
//    contiguous for the other passes (the dgrads 4-8% slower otherwise).
__host__ __forceinline__ int row_map(int mode, int64_t R, int E) {
    if (R > 1024LL * E) return ROW_SHARED;
    const bool fwd = mode == GG_FWD_GATEUP || mode == GG_FWD_DOWN;
    if (R > 640LL * E) return fwd ? ROW_CHUNKED : ROW_SHARED;
    return mode == GG_FWD_GATEUP ? ROW_SHARED : ROW_CONTIGUOUS;
}

// n-tiles of a row-segmented pass (modes GG_FWD_GATEUP .. GG_DGRAD_GATEUP).
__host__ __device__ __forceinline__ int row_n_tiles(int mode, int d, int f) {
    return mode == GG_FWD_GATEUP ? f / 128
         : mode == GG_FWD_DOWN ? d / BN
         : mode == GG_DGRAD_DOWN ? f / BN
         : d / BN;
}

// Weight-gradient output [Mo, No] per expert: dW_d is [f, d]; [dW_g | dW_u] is [d, 2f].
__host__ __device__ __forceinline__ void wgrad_dims(int mode, int d, int f, int& MT, int& NT) {
    MT = (mode == GG_WGRAD_DOWN ? f : d) / BM;
    NT = (mode == GG_WGRAD_DOWN ? d : 2 * f) / BN;
}

// Weight gradients: a tile's K is its expert's segment, which differs between experts (up
// to 15x on skewed routings), so XCD x takes the same contiguous eighth of every expert's
// tile order, [x per / 8, (x + 1) per / 8): every XCD then has the same work whatever the
// segment lengths.  Block b runs the (b / 8)-th tile of its XCD's sequence (expert-major).
// False for a block with no tile.
__host__ __device__ __forceinline__ bool wgrad_tile(int b, int E, int MT, int NT, int& e,
                                                    int& mi, int& ni) {
    const int per = MT * NT;
    const int x = b % NXCD, j = b / NXCD;
    const int lo = (int)((int64_t)x * per / NXCD);
    const int cnt = (int)((int64_t)(x + 1) * per / NXCD) - lo;
    if (cnt == 0) return false;
    e = j / cnt;
    if (e >= E) return false;
    grouped_mn(lo + (j - e * cnt), MT, NT, mi, ni);
    return true;
}

// Blocks a pass launches (a multiple of 8): row passes are sized for the worst case of
// ceil(R / 256) + E m-tiles (the real counts live on the device), rounded up to whole
// rounds of eight chunks with the chunked map and plus E blocks per XCD (the rounding of
// each segment's eighth up to whole tiles) with the shared map; the weight gradients for
// ceil(per / 8) tiles of each expert on every XCD.  `map` < 0: the map row_map picks.
__host__ __forceinline__ int64_t grid_blocks(int mode, int E, int64_t R, int d, int f,
                                             int map = -1) {
    int64_t tiles;
    if (mode == GG_WGRAD_DOWN || mode == GG_WGRAD_GATEUP) {
        int MT, NT;
        wgrad_dims(mode, d, f, MT, NT);
        tiles = (int64_t)E * (((int64_t)MT * NT + NXCD - 1) / NXCD) * NXCD;
    } else {
        const int64_t mt_max = (R + BM - 1) / BM + E;
        tiles = mt_max * row_n_tiles(mode, d, f);
        if (map < 0) map = row_map(mode, R, E);
        if (map == ROW_CHUNKED) tiles = (tiles + NXCD * CHUNK - 1) / (NXCD * CHUNK) * (NXCD * CHUNK);
        if (map == ROW_SHARED) tiles = (tiles + NXCD - 1) / NXCD * NXCD + (int64_t)NXCD * E;
    }
    return (tiles + NXCD - 1) / NXCD * NXCD;
}

}  // namespace tiles
}  // namespace moe
