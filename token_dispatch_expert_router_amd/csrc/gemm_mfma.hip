// Grouped GEMMs of the SwiGLU experts on the bf16 matrix cores of gfx950.
//
// "MoE Parallel Folding" (arXiv 2504.14960), knowledge-base notes page, method
// paragraph ("expert FFN computation" between permutation and un-permutation; the
// backward pass runs the duals).  The experts' rows are contiguous segments
// [offsets[e], offsets[e+1]) of the permuted buffer whose sizes live only in device
// memory, so every block finds its (expert, tile) from `offsets` itself: no host
// synchronisation.
//
// One kernel template serves the six passes:
//   FWD_GATEUP   [a | b] = xp [W_g,e | W_u,e], epilogue h = silu(a) * b
//   FWD_DOWN     o = h W_d,e
//   DGRAD_DOWN   dh = d_o W_d,e^T, epilogue da = dh b sig(a)(1 + a(1 - sig(a))), db = dh silu(a)
//   DGRAD_GATEUP dxp = da W_g,e^T + db W_u,e^T        (K = 2f)
//   WGRAD_DOWN   dW_d,e = h_e^T d_o,e                  (K = the segment's rows)
//   WGRAD_GATEUP dW_g,e = xp_e^T da_e, dW_u,e = xp_e^T db_e
//
// Tiling: 256 x 256 output tile, k-step 64, 256 threads = 4 waves in a 2 x 2 grid,
// each wave 128 x 128 = 4 x 4 v_mfma_f32_32x32x16_bf16 tiles (256 fp32 accumulators
// per lane, one wave per SIMD).  Both operand tiles sit in LDS as [256 rows][64 k]
// (k contiguous, 16-byte chunks XOR-swizzled by row) in two stages (128 KB), so each
// MFMA operand is one 16-byte LDS read.  Operands whose contiguous dimension is M or N
// rather than K are transposed in registers (8 x 8 bf16 blocks) on their way to LDS.
// Blocks are dispatched round-robin over the 8 XCDs; logical tiles are remapped so
// that each XCD runs a contiguous range, and consecutive tiles share their weight
// tile (M fastest), which then stays in that XCD's L2.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int TILE = BM * BK;  // elements of one operand tile

__device__ __forceinline__ int xcd_remap(int b, int G8) {
    return (b & 7) * (G8 >> 3) + (b >> 3);
}

// (expert, m-tile, n-tile) of logical tile L for passes with segmented rows.
__device__ __forceinline__ bool decode_rows(int L, const int32_t* __restrict__ offsets, int E,
                                            int n_tiles, int& e, int& m0, int& m_lim, int& nt) {
    int acc = 0;
    for (int i = 0; i < E; ++i) {
        const int lo = offsets[i], hi = offsets[i + 1];
        const int mt = (hi - lo + BM - 1) / BM;
        const int tiles = mt * n_tiles;
        if (L < acc + tiles) {
            const int loc = L - acc;
            e = i;
            m0 = lo + (loc % mt) * BM;
            m_lim = hi;
            nt = loc / mt;
            return true;
        }
        acc += tiles;
    }
    return false;
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Operand stored [rows][K] with K contiguous: thread loads rows rb+32i, chunk ch.
__device__ __forceinline__ void load_rowk(u32x4 (&r)[8], const bf16_t* __restrict__ base,
                                          int64_t ld, int row0, int row_lim, int k0) {
    const int ch = threadIdx.x & 7, rb = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = row0 + rb + 32 * i;
        r[i] = row < row_lim ? *(const u32x4*)(base + (int64_t)row * ld + k0 + ch * 8) : zero4();
    }
}

__device__ __forceinline__ void store_rowk(bf16_t* lds, const u32x4 (&r)[8]) {
    const int ch = threadIdx.x & 7, rb = threadIdx.x >> 3;
    const int pc = ch ^ (rb & 7);
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4*)(lds + (rb + 32 * i) * BK + pc * 8) = r[i];
}

// Operand stored [K][cols] with cols contiguous: thread loads k rows kb*8+i of its
// 8-column block; colptr already points at that block.
__device__ __forceinline__ void load_kmaj(u32x4 (&r)[8], const bf16_t* __restrict__ colptr,
                                          int64_t ld, int k0, int k_lim) {
    const int kb = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int k = k0 + kb * 8 + i;
        r[i] = k < k_lim ? *(const u32x4*)(colptr + (int64_t)k * ld) : zero4();
    }
}

__device__ __forceinline__ uint32_t dw_of(const u32x4& v, int q) {
    return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
}
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
    return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xFFFF0000u);
}

// Transpose the 8 (k) x 8 (col) block and store column j as LDS row cb*8+j.
__device__ __forceinline__ void store_kmaj(bf16_t* lds, const u32x4 (&r)[8]) {
    const int kb = threadIdx.x & 7, cb = threadIdx.x >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int q = j >> 1;
        u32x4 w;
        if ((j & 1) == 0) {
            w.x = lo_pair(dw_of(r[0], q), dw_of(r[1], q));
            w.y = lo_pair(dw_of(r[2], q), dw_of(r[3], q));
            w.z = lo_pair(dw_of(r[4], q), dw_of(r[5], q));
            w.w = lo_pair(dw_of(r[6], q), dw_of(r[7], q));
        } else {
            w.x = hi_pair(dw_of(r[0], q), dw_of(r[1], q));
            w.y = hi_pair(dw_of(r[2], q), dw_of(r[3], q));
            w.z = hi_pair(dw_of(r[4], q), dw_of(r[5], q));
            w.w = hi_pair(dw_of(r[6], q), dw_of(r[7], q));
        }
        const int row = cb * 8 + j;
        *(u32x4*)(lds + row * BK + ((kb ^ j) * 8)) = w;
    }
}

__device__ __forceinline__ bf16x8_t lds_frag(const bf16_t* lds, int row, int chunk) {
    const int pc = chunk ^ (row & 7);
    return __builtin_bit_cast(bf16x8_t, *(const u32x4*)(lds + row * BK + pc * 8));
}

__device__ __forceinline__ float fast_sigmoid(float a) { return 1.0f / (1.0f + __expf(-a)); }

template <int MODE>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
gg_mfma_kernel(GemmArgs g, int total_tiles) {
    __shared__ __attribute__((aligned(16))) bf16_t lds[2][2][TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    if (L >= total_tiles) return;

    const int d = g.d, f = g.f;
    int e = 0, m0 = 0, m_lim = 0, n0 = 0, k_lo = 0, k_hi = 0, nk = 0;
    if (MODE <= GG_DGRAD_GATEUP) {
        const int n_tiles = MODE == GG_FWD_GATEUP ? f / 128
                          : MODE == GG_FWD_DOWN ? d / BN
                          : MODE == GG_DGRAD_DOWN ? f / BN
                          : d / BN;
        int nt;
        if (!decode_rows(L, g.offsets, g.E, n_tiles, e, m0, m_lim, nt)) return;
        n0 = nt * (MODE == GG_FWD_GATEUP ? 128 : BN);
        const int K = MODE == GG_FWD_GATEUP ? d : MODE == GG_FWD_DOWN ? f
                    : MODE == GG_DGRAD_DOWN ? d : 2 * f;
        nk = K / BK;
    } else {
        const int Mo = MODE == GG_WGRAD_DOWN ? f : d;
        const int No = MODE == GG_WGRAD_DOWN ? d : 2 * f;
        const int MT = Mo / BM, NTl = No / BN;
        const int per = MT * NTl;
        e = L / per;
        const int loc = L - e * per;
        m0 = (loc % MT) * BM;
        n0 = (loc / MT) * BN;
        k_lo = g.offsets[e];
        k_hi = g.offsets[e + 1];
        nk = (k_hi - k_lo + BK - 1) / BK;
    }

    const bf16_t* A0 = (const bf16_t*)g.A0;
    const bf16_t* A1 = (const bf16_t*)g.A1;
    const bf16_t* B0 = (const bf16_t*)g.B0;
    const bf16_t* B1 = (const bf16_t*)g.B1;
    const int cb = tid >> 3;  // this thread's 8-column block for k-major loads

    auto load_tiles = [&](int kt, u32x4 (&ra)[8], u32x4 (&rb)[8]) {
        if (MODE == GG_FWD_GATEUP) {
            const int64_t eo = (int64_t)e * d * f;
            load_rowk(ra, A0, d, m0, m_lim, kt * BK);
            const bf16_t* cp = cb < 16 ? B0 + eo + n0 + cb * 8 : B1 + eo + n0 + (cb - 16) * 8;
            load_kmaj(rb, cp, f, kt * BK, d);
        } else if (MODE == GG_FWD_DOWN) {
            load_rowk(ra, A0, f, m0, m_lim, kt * BK);
            load_kmaj(rb, B0 + (int64_t)e * f * d + n0 + cb * 8, d, kt * BK, f);
        } else if (MODE == GG_DGRAD_DOWN) {
            load_rowk(ra, A0, d, m0, m_lim, kt * BK);
            load_rowk(rb, B0 + (int64_t)e * f * d, d, n0, f, kt * BK);
        } else if (MODE == GG_DGRAD_GATEUP) {
            const int kh = f / BK;
            const bool first = kt < kh;
            const int k0 = (first ? kt : kt - kh) * BK;
            load_rowk(ra, first ? A0 : A1, f, m0, m_lim, k0);
            load_rowk(rb, (first ? B0 : B1) + (int64_t)e * d * f, f, n0, d, k0);
        } else if (MODE == GG_WGRAD_DOWN) {
            load_kmaj(ra, A0 + m0 + cb * 8, f, k_lo + kt * BK, k_hi);
            load_kmaj(rb, B0 + n0 + cb * 8, d, k_lo + kt * BK, k_hi);
        } else {  // GG_WGRAD_GATEUP
            load_kmaj(ra, A0 + m0 + cb * 8, d, k_lo + kt * BK, k_hi);
            const bool first = n0 < f;
            load_kmaj(rb, (first ? B0 : B1) + (first ? n0 : n0 - f) + cb * 8, f, k_lo + kt * BK,
                      k_hi);
        }
    };
    auto store_tiles = [&](int st, const u32x4 (&ra)[8], const u32x4 (&rb)[8]) {
        constexpr bool a_kmaj = MODE == GG_WGRAD_DOWN || MODE == GG_WGRAD_GATEUP;
        constexpr bool b_kmaj = MODE == GG_FWD_GATEUP || MODE == GG_FWD_DOWN || a_kmaj;
        if (a_kmaj) store_kmaj(lds[st][0], ra); else store_rowk(lds[st][0], ra);
        if (b_kmaj) store_kmaj(lds[st][1], rb); else store_rowk(lds[st][1], rb);
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // B-tile row of fragment j for this wave (gate/up: gate rows 0..127, up 128..255).
    auto brow = [&](int j) {
        if (MODE == GG_FWD_GATEUP)
            return (j < 2 ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32) + (lane & 31);
        return wn * 128 + j * 32 + (lane & 31);
    };

    if (nk > 0) {
        u32x4 ra[8], rb[8];
        load_tiles(0, ra, rb);
        store_tiles(0, ra, rb);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int st = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) load_tiles(kt + 1, ra, rb);
            const bf16_t* As = lds[st][0];
            const bf16_t* Bs = lds[st][1];
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                const int ch = ks * 2 + (lane >> 5);
                bf16x8_t af[4], bfr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) af[i] = lds_frag(As, wm * 128 + i * 32 + (lane & 31), ch);
#pragma unroll
                for (int j = 0; j < 4; ++j) bfr[j] = lds_frag(Bs, brow(j), ch);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],
                                                                            acc[i][j], 0, 0, 0);
            }
            if (more) store_tiles(st ^ 1, ra, rb);
            __syncthreads();
        }
    }

    // Epilogue.  32x32 MFMA result: lane holds column (lane & 31) and rows
    // 8*(r/4) + 4*(lane/32) + (r%4) for accumulator register r.
    const int cl = lane & 31;
    const int rq = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rl = wm * 128 + i * 32 + 8 * (r >> 2) + rq + (r & 3);
            if (MODE == GG_FWD_GATEUP) {
                const int row = m0 + rl;
                if (row < m_lim) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int col = n0 + wn * 64 + j * 32 + cl;
                        const float a = acc[i][j][r], b = acc[i][j + 2][r];
                        const float h = a * fast_sigmoid(a) * b;
                        const int64_t o = (int64_t)row * f + col;
                        ((bf16_t*)g.C0)[o] = f32_to_bf16(a);
                        ((bf16_t*)g.C1)[o] = f32_to_bf16(b);
                        ((bf16_t*)g.C2)[o] = f32_to_bf16(h);
                    }
                }
            } else if (MODE == GG_FWD_DOWN || MODE == GG_DGRAD_GATEUP) {
                const int row = m0 + rl;
                if (row < m_lim) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int col = n0 + wn * 128 + j * 32 + cl;
                        ((bf16_t*)g.C0)[(int64_t)row * d + col] = f32_to_bf16(acc[i][j][r]);
                    }
                }
            } else if (MODE == GG_DGRAD_DOWN) {
                const int row = m0 + rl;
                if (row < m_lim) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int col = n0 + wn * 128 + j * 32 + cl;
                        const int64_t o = (int64_t)row * f + col;
                        const float dh = acc[i][j][r];
                        const float a = bf16_to_f32(((const bf16_t*)g.X0)[o]);
                        const float b = bf16_to_f32(((const bf16_t*)g.X1)[o]);
                        const float sg = fast_sigmoid(a);
                        ((bf16_t*)g.C0)[o] = f32_to_bf16(dh * b * sg * (1.0f + a * (1.0f - sg)));
                        ((bf16_t*)g.C1)[o] = f32_to_bf16(dh * a * sg);
                    }
                }
            } else if (MODE == GG_WGRAD_DOWN) {
                const int64_t base = (int64_t)e * f * d;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = n0 + wn * 128 + j * 32 + cl;
                    ((bf16_t*)g.C0)[base + (int64_t)(m0 + rl) * d + col] = f32_to_bf16(acc[i][j][r]);
                }
            } else {  // GG_WGRAD_GATEUP
                const int64_t base = (int64_t)e * d * f;
                const bool first = n0 < f;
                bf16_t* out = (bf16_t*)(first ? g.C0 : g.C1);
                const int c0 = first ? n0 : n0 - f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = c0 + wn * 128 + j * 32 + cl;
                    out[base + (int64_t)(m0 + rl) * f + col] = f32_to_bf16(acc[i][j][r]);
                }
            }
        }
    }
}

}  // namespace

bool mfma_shape_ok(const moe_desc& d) {
    return d.dtype == MOE_BF16 && d.d % 256 == 0 && d.f % 256 == 0 && d.d > 0 && d.f > 0;
}

hipError_t launch_gemm_mfma(GemmMode mode, const GemmArgs& a, hipStream_t s) {
    int64_t tiles;
    const int64_t mt_max = (a.R + BM - 1) / BM + a.E;  // row tiles over all segments
    switch (mode) {
        case GG_FWD_GATEUP: tiles = mt_max * (a.f / 128); break;
        case GG_FWD_DOWN: tiles = mt_max * (a.d / BN); break;
        case GG_DGRAD_DOWN: tiles = mt_max * (a.f / BN); break;
        case GG_DGRAD_GATEUP: tiles = mt_max * (a.d / BN); break;
        case GG_WGRAD_DOWN: tiles = (int64_t)a.E * (a.f / BM) * (a.d / BN); break;
        default: tiles = (int64_t)a.E * (a.d / BM) * (2 * a.f / BN); break;
    }
    if (tiles <= 0) return hipSuccess;
    const int64_t g8 = (tiles + 7) / 8 * 8;
    if (g8 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    // Segmented passes decode their tile from offsets; any L beyond the real tiles exits.
    const int total = (mode <= GG_DGRAD_GATEUP) ? (int)tiles : (int)tiles;
    switch (mode) {
        case GG_FWD_GATEUP: gg_mfma_kernel<GG_FWD_GATEUP><<<(unsigned)g8, 256, 0, s>>>(a, total); break;
        case GG_FWD_DOWN: gg_mfma_kernel<GG_FWD_DOWN><<<(unsigned)g8, 256, 0, s>>>(a, total); break;
        case GG_DGRAD_DOWN: gg_mfma_kernel<GG_DGRAD_DOWN><<<(unsigned)g8, 256, 0, s>>>(a, total); break;
        case GG_DGRAD_GATEUP: gg_mfma_kernel<GG_DGRAD_GATEUP><<<(unsigned)g8, 256, 0, s>>>(a, total); break;
        case GG_WGRAD_DOWN: gg_mfma_kernel<GG_WGRAD_DOWN><<<(unsigned)g8, 256, 0, s>>>(a, total); break;
        default: gg_mfma_kernel<GG_WGRAD_GATEUP><<<(unsigned)g8, 256, 0, s>>>(a, total); break;
    }
    return hipGetLastError();
}

}  // namespace moe
