// Grouped GEMMs of the SwiGLU experts on the bf16 matrix cores of gfx950.
//
// "MoE Parallel Folding" (arXiv 2504.14960), knowledge-base notes page, method
// paragraph: the experts' FFNs run on the permuted rows, between permutation and
// un-permutation, and the backward pass runs their duals.  The experts' rows are
// contiguous segments [offsets[e], offsets[e+1]) of the permuted buffer whose sizes
// live only in device memory, so every block finds its (expert, tile) from `offsets`
// itself: no host synchronisation.
//
// One kernel template serves the six passes:
//   FWD_GATEUP   [a | b] = xp [W_g,e | W_u,e], epilogue h = silu(a) * b
//   FWD_DOWN     o = h W_d,e
//   DGRAD_DOWN   dh = d_o W_d,e^T, epilogue da = dh b sig(a)(1 + a(1 - sig(a))), db = dh silu(a)
//   DGRAD_GATEUP dxp = da W_g,e^T + db W_u,e^T        (K = 2f)
//   WGRAD_DOWN   dW_d,e = h_e^T d_o,e                  (K = the segment's rows)
//   WGRAD_GATEUP dW_g,e = xp_e^T da_e, dW_u,e = xp_e^T db_e
//
// Tiling.  256 x 256 output tile, k-step 32, 256 threads = 4 waves in a 2 x 2 grid,
// each wave 128 x 128 = 4 x 4 v_mfma_f32_32x32x16_bf16 tiles (256 fp32 accumulators
// per lane in AGPRs, one wave per SIMD).
//
// Data path.  Operand tiles go from global memory straight into LDS with
// global_load_lds_dwordx4 (no register staging, no LDS store instructions), in a
// 4-stage ring of 32 KB stages (128 KB), three k-steps in flight.  An operand whose
// contiguous dimension is K sits in LDS as [256 rows][32 k] and a fragment is one
// ds_read_b128; an operand whose contiguous dimension is M or N sits as it is in
// memory, [32 k][256 cols], and a fragment is two ds_read_b64_tr_b16 (the LDS
// transpose read of gfx950: in each 16-lane group, lane i receives element i%4 of the
// 8 bytes addressed by lane 4j + i/4, for j = 0..3).  Both layouts XOR-swizzle their
// 16-byte chunks so that the fragment reads are free of bank conflicts; the swizzle is
// applied by choosing which global chunk each lane fetches, since a direct load
// writes its 64 lanes' 16 bytes to 1 KB of consecutive LDS.
//
// Schedule per k-step: read the fragments of sub-step 1, issue the 16 MFMAs of
// sub-step 0, wait for the next stage and pass the barrier, refill the freed stage,
// read the fragments of the next stage's sub-step 0, issue the 16 MFMAs of sub-step 1.
// MFMAs already issued keep the matrix pipe busy while the wave waits at the barrier.
//
// Blocks are dispatched round-robin over the 8 XCDs; logical tiles are remapped so
// that each XCD runs a contiguous range, in which consecutive tiles share their
// weight tile (M fastest) and stay in that XCD's L2.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;
constexpr int STAGES = 4;
constexpr int TILE_BYTES = BM * BK * 2;          // one operand tile of one stage: 16 KB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;      // A and B

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

// Swizzles.  K-major tile [256][32]: physical chunk p of row r holds logical chunk
// p ^ swz_k(r).  MN-major tile [32][256]: physical chunk p of k-row r holds logical
// chunk p ^ swz_mn(r).  gfx950 serves a ds_read_b128 16 consecutive lanes at a time
// over 64 four-byte banks; with these swizzles the fragment reads of both layouts
// measure free of bank conflicts (SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int swz_k(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz_mn(int r) { return (r & 3) << 2; }

// Direct global -> LDS load of 16 bytes per lane (the 64 lanes fill 1 KB of LDS
// starting at lds_addr, which must be wave-uniform).  Written as inline asm so that
// the compiler does not treat every later LDS read as possibly aliasing it (it would
// wait for all loads in flight before each read); completion is awaited explicitly
// with s_waitcnt vmcnt before the barrier that publishes a stage.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds_addr) : "memory", "m0");
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// LDS fragment reads.  The compiler sees these as LDS loads and places the waits
// for their results itself.
__device__ __forceinline__ void ds_b128(u32x4_t& v, uint32_t addr) {
    v = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)addr;
}
__device__ __forceinline__ void ds_tr_pair(s16x4_t& lo, s16x4_t& hi, uint32_t addr) {
    lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr);
    hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(addr + 2048));
}

// Byte address of a K-major fragment: row of the tile, 16-byte chunk.
__device__ __forceinline__ uint32_t addr_k(uint32_t tile, int row, int chunk) {
    return tile + row * 64 + ((chunk ^ swz_k(row)) << 4);
}
// Byte address of the first of the two transpose reads of an MN-major fragment:
// columns [c0, c0+32) of the tile, k rows 16*ks + [0, 16); the second read is 4 k rows
// (2048 bytes) further, with the same swizzle.
__device__ __forceinline__ uint32_t addr_mn(uint32_t tile, int c0, int ks, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int col = c0 + 16 * (g & 1) + 4 * (s & 3);
    const int kr = 16 * ks + 8 * (g >> 1) + (s >> 2);
    return tile + kr * 512 + (((col >> 3) ^ swz_mn(kr)) << 4) + (col & 7) * 2;
}

struct Frag {
    s16x4_t lo[4], hi[4];  // MN-major fragments (two transpose reads)
    u32x4_t q[4];          // K-major fragments (one read)
};

template <bool MN>
__device__ __forceinline__ bf16x8_t frag_value(const Frag& f, int i) {
    if (MN) {
        s16x8_t v = __builtin_shufflevector(f.lo[i], f.hi[i], 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8_t, v);
    }
    return __builtin_bit_cast(bf16x8_t, f.q[i]);
}

__device__ __forceinline__ float fast_sigmoid(float a) { return 1.0f / (1.0f + __expf(-a)); }

template <int MODE> struct Traits {
    static constexpr bool a_mn = MODE == GG_WGRAD_DOWN || MODE == GG_WGRAD_GATEUP;
    static constexpr bool b_mn = MODE == GG_FWD_GATEUP || MODE == GG_FWD_DOWN || a_mn;
};

template <int MODE>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
gg_mfma_kernel(GemmArgs g, int total_tiles) {
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
    using TR = Traits<MODE>;

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
    const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;

    // ---- per-lane source offsets (elements) of this wave's 4 direct loads per operand --
    // K-major: instruction i covers tile rows (wave*4+i)*16 + lane/4, physical chunk lane%4.
    // MN-major: instruction i covers k rows (wave*4+i)*2 + lane/32, physical chunk lane%32.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int64_t a_off[4], b_off[4];
    int a_kr[4], b_kr[4];
    bool b_up[4];  // gate/up: this lane's chunk comes from W_u
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b_up[i] = false;
        if (!TR::a_mn) {
            const int row = (wv * 4 + i) * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz_k(row);
            const int grow = min(m0 + row, m_lim - 1);  // rows past the segment: any valid row
            const int64_t lda = (MODE == GG_FWD_GATEUP || MODE == GG_DGRAD_DOWN) ? d : f;
            a_off[i] = (int64_t)grow * lda + c * 8;
            a_kr[i] = 0;
        } else {
            const int kr = (wv * 4 + i) * 2 + (lane >> 5);
            const int c = (lane & 31) ^ swz_mn(kr);
            a_off[i] = m0 + c * 8;
            a_kr[i] = kr;
        }
        if (!TR::b_mn) {
            const int row = (wv * 4 + i) * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz_k(row);
            b_off[i] = MODE == GG_DGRAD_DOWN
                           ? (int64_t)e * f * d + (int64_t)(n0 + row) * d + c * 8
                           : (int64_t)e * d * f + (int64_t)(n0 + row) * f + c * 8;
            b_kr[i] = 0;
        } else {
            const int kr = (wv * 4 + i) * 2 + (lane >> 5);
            const int c = (lane & 31) ^ swz_mn(kr);
            b_kr[i] = kr;
            if (MODE == GG_FWD_GATEUP) {
                b_up[i] = c >= 16;
                b_off[i] = (int64_t)e * d * f + n0 + (c & 15) * 8;
            } else if (MODE == GG_FWD_DOWN) {
                b_off[i] = (int64_t)e * f * d + n0 + c * 8;
            } else if (MODE == GG_WGRAD_DOWN) {
                b_off[i] = n0 + c * 8;
            } else {
                b_off[i] = (n0 < f ? n0 : n0 - f) + c * 8;
            }
        }
    }

    // Issue the i-th direct load of each operand of k-step kt into stage st.
    auto issue_one = [&](int kt, int st, int i) {
        const uint32_t sa = smem_base + st * STAGE_BYTES + wv * 4 * 1024;
        const uint32_t sb = sa + TILE_BYTES;
        const int k0 = kt * BK;
        const bool first_half = k0 < f;            // gate/up dgrad: da, W_g then db, W_u
        const int kh = first_half ? k0 : k0 - f;
        {
            const bf16_t* pa;
            const bf16_t* pb;
            if (MODE == GG_FWD_GATEUP || MODE == GG_FWD_DOWN || MODE == GG_DGRAD_DOWN) {
                pa = A0 + a_off[i] + k0;
            } else if (MODE == GG_DGRAD_GATEUP) {
                pa = (first_half ? A0 : A1) + a_off[i] + kh;
            } else {
                const int kr = min(k_lo + k0 + a_kr[i], k_hi - 1);  // tail rows zeroed later
                pa = A0 + a_off[i] + (int64_t)kr * (MODE == GG_WGRAD_DOWN ? f : d);
            }
            if (MODE == GG_DGRAD_DOWN) {
                pb = B0 + b_off[i] + k0;
            } else if (MODE == GG_DGRAD_GATEUP) {
                pb = (first_half ? B0 : B1) + b_off[i] + kh;
            } else if (MODE == GG_FWD_GATEUP) {
                pb = (b_up[i] ? B1 : B0) + b_off[i] + (int64_t)(k0 + b_kr[i]) * f;
            } else if (MODE == GG_FWD_DOWN) {
                pb = B0 + b_off[i] + (int64_t)(k0 + b_kr[i]) * d;
            } else {
                const int kr = min(k_lo + k0 + b_kr[i], k_hi - 1);
                pb = (MODE == GG_WGRAD_GATEUP && n0 >= f ? B1 : B0) + b_off[i] +
                     (int64_t)kr * (MODE == GG_WGRAD_DOWN ? d : f);
            }
            lds_dma16(pa, sa + i * 1024);
            lds_dma16(pb, sb + i * 1024);
        }
    };
    auto issue = [&](int kt, int st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) issue_one(kt, st, i);
    };

    // Per-lane LDS byte offsets (within a stage) of this wave's fragment reads.
    uint32_t a_rd[2][4], b_rd[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a_rd[ks][i] = TR::a_mn ? addr_mn(0, wm * 128 + i * 32, ks, lane)
                                   : addr_k(0, wm * 128 + i * 32 + (lane & 31), 2 * ks + (lane >> 5));
            // gate/up: gate columns are tile rows 0..127, up columns 128..255
            const int c0 = MODE == GG_FWD_GATEUP
                               ? (i < 2 ? wn * 64 + i * 32 : 128 + wn * 64 + (i - 2) * 32)
                               : wn * 128 + i * 32;
            b_rd[ks][i] = TR::b_mn ? addr_mn(TILE_BYTES, c0, ks, lane)
                                   : addr_k(TILE_BYTES, c0 + (lane & 31), 2 * ks + (lane >> 5));
        }
    }
    // The r-th read of a sub-step's fragments: A fragments first, then B.
    auto read_op = [&](int r, uint32_t stage, int ks, Frag& fa, Frag& fb) {
        if (TR::a_mn) {
            if (r < 4) ds_tr_pair(fa.lo[r], fa.hi[r], stage + a_rd[ks][r]);
        } else {
            if (r < 4) ds_b128(fa.q[r], stage + a_rd[ks][r]);
        }
        if (r >= 4 && r < 8) {
            const int j = r - 4;
            if (TR::b_mn) ds_tr_pair(fb.lo[j], fb.hi[j], stage + b_rd[ks][j]);
            else ds_b128(fb.q[j], stage + b_rd[ks][j]);
        }
    };

    // Rows [valid, 32) of the A tile of stage st hold clamped copies: zero them (wgrad K tail).
    auto zero_tail = [&](int st, int valid) {
        const uint32_t ta = smem_base + st * STAGE_BYTES;
        for (int idx = tid; idx < (BK - valid) * 32; idx += 256) {
            const int r = valid + idx / 32, c = idx % 32;
            *(__attribute__((address_space(3))) u32x4_t*)(uintptr_t)(ta + r * 512 + c * 16) =
                u32x4_t{0u, 0u, 0u, 0u};
        }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int tail_valid = TR::a_mn ? (k_hi - k_lo) - (nk - 1) * BK : BK;

    if (nk > 0) {
        Frag f0a, f0b, f1a, f1b;  // sub-step 0 and sub-step 1 fragments
        issue(0, 0);
        if (nk > 1) issue(1, 1);
        if (nk > 2) issue(2, 2);
        if (nk > 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else if (nk > 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        if (TR::a_mn && nk == 1 && tail_valid < BK) {
            zero_tail(0, tail_valid);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) read_op(r, smem_base, 0, f0a, f0b);

        for (int kt = 0; kt < nk; ++kt) {
            const int st = kt & (STAGES - 1);
            const uint32_t stage = smem_base + st * STAGE_BYTES;
            const bool more = kt + 1 < nk;
            const uint32_t next = smem_base + ((kt + 1) & (STAGES - 1)) * STAGE_BYTES;

            // Phase A: MFMAs of sub-step 0, with the reads of sub-step 1 between them.
            // One MFMA and one read per slot, fenced so the compiler keeps the order.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int i = q >> 2, j = q & 3;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    frag_value<TR::a_mn>(f0a, i), frag_value<TR::b_mn>(f0b, j), acc[i][j], 0, 0, 0);
                if (q < 8) read_op(q, stage, 1, f1a, f1b);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (more) {
                // the loads of k-step kt+1 have landed in this wave; after the barrier, in all
                if (kt + 2 < nk) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                if (TR::a_mn && kt + 2 == nk && tail_valid < BK) {
                    zero_tail((kt + 1) & (STAGES - 1), tail_valid);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                }
            }
            // Phase B: MFMAs of sub-step 1, with the reads of the next stage's sub-step 0
            // and the refill of the stage freed by the previous k-step between them.  After
            // the last k-step the reads touch a stage nobody uses: in bounds, and unused.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int i = q >> 2, j = q & 3;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    frag_value<TR::a_mn>(f1a, i), frag_value<TR::b_mn>(f1b, j), acc[i][j], 0, 0, 0);
                if (q < 8) read_op(q, next, 0, f0a, f0b);
                else if (q < 12 && kt + 3 < nk) issue_one(kt + 3, (kt + 3) & (STAGES - 1), q - 8);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    // Epilogue.  32x32 MFMA result: lane holds column (lane & 31) and rows
    // 8*(r/4) + 4*(lane/32) + (r%4) for accumulator register r.  Each wave stages one
    // 32-row band of its fp32 results at a time in a private 32 KB of LDS, then every
    // lane handles 8-column chunks: 16-byte coalesced loads of epilogue inputs and
    // 16-byte stores (16 lanes cover 256 contiguous bytes of a row).
    __builtin_amdgcn_s_barrier();  // every wave is done reading the operand stages
    typedef __attribute__((address_space(3))) float lds_f32;
    const uint32_t wbase = smem_base + wv * 32768;
    const int cl = lane & 31;
    const int rq = 4 * (lane >> 5);
    constexpr int P = MODE == GG_FWD_GATEUP ? 68 : 132;  // band row pitch in floats
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // gate/up: columns j = 0, 1 are a (first buffer), j = 2, 3 are b (second)
            const uint32_t buf = (MODE == GG_FWD_GATEUP && j >= 2) ? wbase + 32 * P * 4 : wbase;
            const int col = (MODE == GG_FWD_GATEUP ? (j & 1) : j) * 32 + cl;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = 8 * (r >> 2) + rq + (r & 3);
                *(lds_f32*)(uintptr_t)(buf + (rl * P + col) * 4) = acc[i][j][r];
            }
        }
        const int row_base = wm * 128 + i * 32;  // within the block tile
        if (MODE == GG_FWD_GATEUP) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int q = lane + 64 * t;
                const int rl = q >> 3, cc = q & 7;
                const int row = m0 + row_base + rl;
                const uint32_t la = wbase + (rl * P + cc * 8) * 4;
                const uint32_t lb = la + 32 * P * 4;
                u32x4_t a0 = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)la;
                u32x4_t a1 = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(la + 16);
                u32x4_t b0 = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)lb;
                u32x4_t b1 = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(lb + 16);
                if (row < m_lim) {
                    float av[8], bv[8], hv[8];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        av[u] = __uint_as_float(a0[u]); av[u + 4] = __uint_as_float(a1[u]);
                        bv[u] = __uint_as_float(b0[u]); bv[u + 4] = __uint_as_float(b1[u]);
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) hv[u] = av[u] * fast_sigmoid(av[u]) * bv[u];
                    const int64_t o = (int64_t)row * f + n0 + wn * 64 + cc * 8;
                    *(u32x4*)((bf16_t*)g.C0 + o) = Vec16<bf16_t>::pack(av);
                    *(u32x4*)((bf16_t*)g.C1 + o) = Vec16<bf16_t>::pack(bv);
                    *(u32x4*)((bf16_t*)g.C2 + o) = Vec16<bf16_t>::pack(hv);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int q = lane + 64 * t;
                const int rl = q >> 4, cc = q & 15;
                const uint32_t la = wbase + (rl * P + cc * 8) * 4;
                u32x4_t v0 = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)la;
                u32x4_t v1 = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(la + 16);
                float v[8];
#pragma unroll
                for (int u = 0; u < 4; ++u) { v[u] = __uint_as_float(v0[u]); v[u + 4] = __uint_as_float(v1[u]); }
                const int rt = row_base + rl;              // row within the block tile
                const int ct = wn * 128 + cc * 8;          // column within the block tile
                if (MODE == GG_FWD_DOWN || MODE == GG_DGRAD_GATEUP) {
                    const int row = m0 + rt;
                    if (row < m_lim)
                        *(u32x4*)((bf16_t*)g.C0 + (int64_t)row * d + n0 + ct) = Vec16<bf16_t>::pack(v);
                } else if (MODE == GG_DGRAD_DOWN) {
                    const int row = m0 + rt;
                    if (row < m_lim) {
                        const int64_t o = (int64_t)row * f + n0 + ct;
                        float av[8], bv[8], dav[8], dbv[8];
                        Vec16<bf16_t>::unpack(*(const u32x4*)((const bf16_t*)g.X0 + o), av);
                        Vec16<bf16_t>::unpack(*(const u32x4*)((const bf16_t*)g.X1 + o), bv);
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const float sg = fast_sigmoid(av[u]);
                            dav[u] = v[u] * bv[u] * sg * (1.0f + av[u] * (1.0f - sg));
                            dbv[u] = v[u] * av[u] * sg;
                        }
                        *(u32x4*)((bf16_t*)g.C0 + o) = Vec16<bf16_t>::pack(dav);
                        *(u32x4*)((bf16_t*)g.C1 + o) = Vec16<bf16_t>::pack(dbv);
                    }
                } else if (MODE == GG_WGRAD_DOWN) {
                    const int64_t o = (int64_t)e * f * d + (int64_t)(m0 + rt) * d + n0 + ct;
                    *(u32x4*)((bf16_t*)g.C0 + o) = Vec16<bf16_t>::pack(v);
                } else {  // GG_WGRAD_GATEUP
                    const bool first = n0 < f;
                    bf16_t* out = (bf16_t*)(first ? g.C0 : g.C1);
                    const int64_t o = (int64_t)e * d * f + (int64_t)(m0 + rt) * f +
                                      (first ? n0 : n0 - f) + ct;
                    *(u32x4*)(out + o) = Vec16<bf16_t>::pack(v);
                }
            }
        }
    }
}

template <int MODE>
hipError_t launch_mode(const GemmArgs& a, unsigned g8, int total, hipStream_t s) {
    gg_mfma_kernel<MODE><<<g8, 256, 0, s>>>(a, total);
    return hipGetLastError();
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
    const unsigned G = (unsigned)g8;
    const int total = (int)tiles;
    switch (mode) {
        case GG_FWD_GATEUP: return launch_mode<GG_FWD_GATEUP>(a, G, total, s);
        case GG_FWD_DOWN: return launch_mode<GG_FWD_DOWN>(a, G, total, s);
        case GG_DGRAD_DOWN: return launch_mode<GG_DGRAD_DOWN>(a, G, total, s);
        case GG_DGRAD_GATEUP: return launch_mode<GG_DGRAD_GATEUP>(a, G, total, s);
        case GG_WGRAD_DOWN: return launch_mode<GG_WGRAD_DOWN>(a, G, total, s);
        default: return launch_mode<GG_WGRAD_GATEUP>(a, G, total, s);
    }
}

}  // namespace moe
