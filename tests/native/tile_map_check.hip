// Host-side check of the grouped GEMM's tile maps (csrc/tile_map.h, the same functions
// the kernels run), over given segment offsets.  For each of the six passes it walks
// every block of the launch grid and checks:
//   - row passes, with and without half-height last tiles: the grid holds every real
//     tile; each block maps to at most one tile, which lies inside one segment (first row
//     in [lo, hi), tile-aligned from lo, limit hi, a 128-row tile only as a segment's
//     last tile reaching its end) with an n-tile in range; every (expert, m-tile, n-tile)
//     is produced exactly once; with the contiguous map each XCD (block b on XCD b % 8)
//     runs one contiguous range of the logical tile order, with the chunked map whole
//     chunks x, x + 8, ... of it, with the shared map the same share of every expert's
//     tiles to within one, one contiguous range of each expert's tile order, expert by
//     expert;
//   - weight gradients: every (expert, m-tile, n-tile) exactly once, and each XCD gets
//     the same share of every expert's tiles to within one.
// Usage: tile_map_check E R d f off_0 ... off_E   (prints one line per pass; exit 1 on
// the first violation).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../../token_dispatch_expert_router_amd/csrc/tile_map.h"

using namespace moe;

static int fail(const char* pass, const char* what, long a, long b, long c) {
    printf("FAIL %s: %s (%ld, %ld, %ld)\n", pass, what, a, b, c);
    return 1;
}

// Position of (m-tile mi, n-tile ni) in a segment's grouped tile order (the inverse of
// tiles::grouped_mn).
static int grouped_pos(int mi, int ni, int mt, int n_tiles) {
    const int gi = mi / tiles::GROUP_M;
    const int rest = mt - gi * tiles::GROUP_M;
    const int gm = rest < tiles::GROUP_M ? rest : tiles::GROUP_M;
    return gi * tiles::GROUP_M * n_tiles + ni * gm + (mi - gi * tiles::GROUP_M);
}

// Every map is walked over the grid sized for it (tiles::grid_blocks with that map); the
// launch takes the one tiles::row_map picks.
static int check_rows(int mode, const char* name, const std::vector<int32_t>& off, int E, int64_t R,
                      int d, int f, bool half, int map) {
    const int nt_n = tiles::row_n_tiles(mode, d, f);
    const int64_t G = tiles::grid_blocks(mode, E, R, d, f, map);
    const bool share = map == tiles::ROW_SHARED;
    const int valid = tiles::count_row_tiles(off.data(), E) * nt_n;
    if (G % 8 != 0) return fail(name, "grid not a multiple of 8", G, 0, 0);
    std::vector<int> seen;
    std::vector<int64_t> base(E + 1, 0);
    for (int e = 0; e < E; ++e)
        base[e + 1] = base[e] + (int64_t)((off[e + 1] - off[e] + tiles::BM - 1) / tiles::BM) * nt_n;
    seen.assign((size_t)base[E], 0);
    std::vector<int> share_n((size_t)E * 8, 0), last_e(8, -1);
    std::vector<int64_t> lo_L(8, INT64_MAX), hi_L(8, -1), n_L(8, 0);
    std::vector<int> lo_p((size_t)E * 8, 1 << 30), hi_p((size_t)E * 8, -1);
    for (int64_t b = 0; b < G; ++b) {
        int e, m0, m_lim, nt, mh;
        if (!tiles::row_tile((int)b, off.data(), E, nt_n, half, map, e, m0, m_lim, nt, mh)) continue;
        if (e < 0 || e >= E) return fail(name, "expert out of range", b, e, E);
        const int lo = off[e], hi = off[e + 1];
        if (!(m0 >= lo && m0 < hi)) return fail(name, "first row outside its segment", e, m0, lo);
        // a tile covers rows [m0, min(m0 + mh, hi)); a half-height tile must reach the
        // segment's end (it is the last one) and only the half-tile launch makes them
        if (mh != tiles::BM && !(half && mh == tiles::BM / 2 && hi - m0 <= mh))
            return fail(name, "bad tile height", e, m0, mh);
        if ((m0 - lo) % tiles::BM) return fail(name, "tile not aligned in its segment", e, m0, lo);
        if (m_lim != hi || hi > R) return fail(name, "row limit", e, m_lim, hi);
        if (nt < 0 || nt >= nt_n) return fail(name, "n-tile out of range", e, nt, nt_n);
        const int x = (int)(b % 8);
        const int mi = (m0 - lo) / tiles::BM, mt = (hi - lo + tiles::BM - 1) / tiles::BM;
        const int pos = grouped_pos(mi, nt, mt, nt_n);
        const int64_t L = base[e] + pos;
        if (map == tiles::ROW_CHUNKED && (L / tiles::CHUNK) % 8 != x)
            return fail(name, "a chunk on the wrong XCD", x, (long)L, (long)(L / tiles::CHUNK));
        lo_L[x] = L < lo_L[x] ? L : lo_L[x];
        hi_L[x] = L > hi_L[x] ? L : hi_L[x];
        n_L[x]++;
        const size_t ex = (size_t)e * 8 + x;
        lo_p[ex] = pos < lo_p[ex] ? pos : lo_p[ex];
        hi_p[ex] = pos > hi_p[ex] ? pos : hi_p[ex];
        if (share && e < last_e[x]) return fail(name, "an XCD's tiles are not expert by expert", x, e, last_e[x]);
        last_e[x] = e;
        share_n[ex]++;
        const int64_t id = base[e] + (int64_t)mi * nt_n + nt;
        if (++seen[(size_t)id] != 1) return fail(name, "tile produced twice", e, m0, nt);
    }
    for (size_t i = 0; i < seen.size(); ++i)
        if (seen[i] != 1) return fail(name, "tile never produced", (long)i, (long)seen.size(), 0);
    if (map == tiles::ROW_CONTIGUOUS) {
        for (int x = 0; x < 8; ++x)
            if (n_L[x] && hi_L[x] - lo_L[x] + 1 != n_L[x])
                return fail(name, "an XCD's tiles are not one contiguous range", x, (long)lo_L[x], (long)hi_L[x]);
    } else if (share) {
        for (int e = 0; e < E; ++e) {
            int mn = 1 << 30, mx = 0;
            for (int x = 0; x < 8; ++x) {
                const size_t ex = (size_t)e * 8 + x;
                const int v = share_n[ex];
                mn = v < mn ? v : mn;
                mx = v > mx ? v : mx;
                if (v && hi_p[ex] - lo_p[ex] + 1 != v)
                    return fail(name, "an XCD's share of an expert is not contiguous", e, x, v);
            }
            if (mx - mn > 1) return fail(name, "uneven XCD share of an expert", e, mn, mx);
        }
    }
    static const char* map_name[3] = {" (contiguous map)", " (shared map)", " (chunked map)"};
    printf("%s%s%s blocks %lld tiles %d ok\n", name, half ? " (half tiles)" : "", map_name[map],
           (long long)G, valid);
    return 0;
}

static int check_wgrad(int mode, const char* name, int E, int64_t R, int d, int f) {
    int MT, NT;
    tiles::wgrad_dims(mode, d, f, MT, NT);
    const int64_t G = tiles::grid_blocks(mode, E, R, d, f);
    std::vector<int> seen((size_t)E * MT * NT, 0);
    std::vector<int> share((size_t)E * 8, 0);
    for (int64_t b = 0; b < G; ++b) {
        int e, mi, ni;
        if (!tiles::wgrad_tile((int)b, E, MT, NT, e, mi, ni)) continue;
        if (e < 0 || e >= E || mi < 0 || mi >= MT || ni < 0 || ni >= NT)
            return fail(name, "tile out of range", e, mi, ni);
        if (++seen[((size_t)e * MT + mi) * NT + ni] != 1)
            return fail(name, "tile produced twice", e, mi, ni);
        share[(size_t)e * 8 + b % 8]++;
    }
    for (size_t i = 0; i < seen.size(); ++i)
        if (seen[i] != 1) return fail(name, "tile never produced", (long)i, 0, 0);
    for (int e = 0; e < E; ++e) {
        int mn = 1 << 30, mx = 0;
        for (int x = 0; x < 8; ++x) {
            const int v = share[(size_t)e * 8 + x];
            mn = v < mn ? v : mn;
            mx = v > mx ? v : mx;
        }
        if (mx - mn > 1) return fail(name, "uneven XCD share of an expert", e, mn, mx);
    }
    // The persistent launch: P blocks (a multiple of 8, at most G), block p walking
    // b = p, p + P, ... and stopping at the first b without a tile; every tile must again
    // be produced exactly once, by a block on the XCD b % 8 of its one-tile-per-block launch.
    for (int P : {256, 64, 8}) {
        const int64_t PP = P < G ? P : G;
        std::vector<int> seen_p((size_t)E * MT * NT, 0);
        for (int64_t p = 0; p < PP; ++p)
            for (int64_t b = p;; b += PP) {
                int e, mi, ni;
                if (b > 0x7FFFFFFF || !tiles::wgrad_tile((int)b, E, MT, NT, e, mi, ni)) break;
                if (b % 8 != p % 8) return fail(name, "persistent walk changed XCD", (long)p, (long)b, 0);
                if (++seen_p[((size_t)e * MT + mi) * NT + ni] != 1)
                    return fail(name, "persistent walk: tile produced twice", e, mi, ni);
            }
        for (size_t i = 0; i < seen_p.size(); ++i)
            if (seen_p[i] != 1) return fail(name, "persistent walk: tile never produced", (long)i, P, 0);
    }
    printf("%s blocks %lld tiles %d ok\n", name, (long long)G, E * MT * NT);
    return 0;
}

int main(int argc, char** argv) {
    if (argc < 6) {
        fprintf(stderr, "usage: %s E R d f off_0 ... off_E\n", argv[0]);
        return 2;
    }
    const int E = atoi(argv[1]);
    const int64_t R = atoll(argv[2]);
    const int d = atoi(argv[3]), f = atoi(argv[4]);
    if (E < 1 || argc != 5 + E + 1 || d % 256 || f % 256) {
        fprintf(stderr, "bad arguments\n");
        return 2;
    }
    std::vector<int32_t> off(E + 1);
    for (int i = 0; i <= E; ++i) off[i] = atoi(argv[5 + i]);
    if (off[0] != 0) return fail("input", "offsets[0] != 0", off[0], 0, 0);
    for (int i = 0; i < E; ++i)
        if (off[i + 1] < off[i]) return fail("input", "offsets decrease", i, off[i], off[i + 1]);
    if (off[E] > R) return fail("input", "offsets[E] > R", off[E], R, 0);
    int rc = 0;
    for (int h = 0; h < 2; ++h)
        for (int map = 0; map < 3; ++map) {
            rc |= check_rows(GG_FWD_GATEUP, "fwd_gateup", off, E, R, d, f, h == 1, map);
            rc |= check_rows(GG_FWD_DOWN, "fwd_down", off, E, R, d, f, h == 1, map);
            rc |= check_rows(GG_DGRAD_DOWN, "dgrad_down", off, E, R, d, f, h == 1, map);
            rc |= check_rows(GG_DGRAD_GATEUP, "dgrad_gateup", off, E, R, d, f, h == 1, map);
        }
    rc |= check_wgrad(GG_WGRAD_DOWN, "wgrad_down", E, R, d, f);
    rc |= check_wgrad(GG_WGRAD_GATEUP, "wgrad_gateup", E, R, d, f);
    return rc;
}
