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
// Tiling.  256 x 256 output tile, k-step 32, 512 threads = 8 waves; wave w computes
// rows 128*(w & 1) .. +127 and columns 64*(w >> 1) .. +63 of the tile as 8 x 4
// v_mfma_f32_16x16x32_bf16 blocks (128 fp32 accumulators per lane, two waves per SIMD).
// A fragment holds 16 rows (columns) x 8 consecutive k per lane group of 16, so one
// k-step is a single 32-deep MFMA per block; with changing operand data the 16x16x32
// form sustains a higher clock than 32x32x16 under the power limit (it reads and
// writes half the accumulator bytes per FLOP).
//
// Data path.  Operand tiles go from global memory straight into LDS with direct
// buffer loads (buffer_load_dwordx4 ... lds: no register staging, no LDS store
// instructions, 32-bit per-lane offsets against a per-tile buffer resource).  An operand
// whose contiguous dimension is K sits in LDS as [256 rows][k] and a fragment is one
// ds_read_b128; an operand whose contiguous dimension is M or N sits as it is in
// memory, [32 k][256 cols], and a fragment is two ds_read_b64_tr_b16 (the LDS
// transpose read of gfx950: in each 16-lane group, lane i receives element i%4 of the
// 8 bytes addressed by lane 4j + i/4, for j = 0..3).  All layouts XOR-swizzle their
// 16-byte chunks so that the fragment reads are free of bank conflicts; the swizzle is
// applied by choosing which global chunk each lane fetches, since a direct load
// writes its 64 lanes' 16 bytes to 1 KB of consecutive LDS.
//
// Staging.  The forward passes and the weight gradients use a 4-stage ring of single
// k-steps (32 KB each, three k-steps in flight).  The two dgrads, whose operands are both
// K-major, load pairs of k-steps into two 64 KB slots instead, so that a K-major row is
// 128 bytes and every load instruction reads whole cache lines (with single k-steps an
// instruction reads 16 rows of 64 bytes).
//
// Schedule (ping-pong).  Waves w and w + 4 share a SIMD.  Waves 0-3 and waves 4-7 run
// the same sequence -- memory phase M(k): read every fragment of k-step k from LDS;
// compute phase C(k): the 32 MFMAs of k-step k with this wave's share of the direct
// loads between them -- one phase apart, separated by block barriers, so that on
// every SIMD one wave issues MFMAs while the other reads LDS.  The LDS reads of one
// phase take about as long as its MFMAs, and the direct loads are issued by the
// computing wave, where their issue cost hides under the MFMA pipeline.  Every k-loop
// runs its steady-state k-steps (refill target in range, fixed wait counts) as a
// separate copy of the loop body with unconditional loads and constant waits, and the
// dgrads and forward passes run one copy of the loop per wave group: the loop's own
// branches cost 2-7% per pass.
//
// Blocks are dispatched round-robin over the 8 XCDs; logical tiles are remapped so
// that each XCD runs contiguous runs of tiles, in which consecutive tiles form 4 x 8
// blocks (groups of four m-tiles, M fastest) whose operand panels stay in that XCD's L2:
// one contiguous eighth of all tiles, chunks of 32 tiles dealt round-robin, or the same
// contiguous eighth of every expert's tiles, chosen per launch by measurement
// (tiles::row_map).  The
// weight-gradient passes, whose tiles' K is their expert's segment length, always take
// the latter; with short segments they run as one persistent block per CU that carries
// the operand ring from tile to tile (gg_wgrad_kernel).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "tile_map.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;
// Two staging schemes share the 128 KB of LDS:
//  - single k-steps: a ring of 4 stages of 32 KB ([A 16 KB | B 16 KB] per k-step);
//  - pairs of k-steps: 2 slots of 64 KB ([A 32 KB | B 32 KB] per 64 k).
constexpr int STEP_STAGES = 4;
constexpr int STEP_TILE_BYTES = BM * BK * 2;            // one operand of one k-step: 16 KB
constexpr int STEP_STAGE_BYTES = 2 * STEP_TILE_BYTES;   // A and B of one k-step
constexpr int KP = 2 * BK;                              // k of one pair
constexpr int OP_BYTES = BM * KP * 2;                   // one operand of one pair: 32 KB
constexpr int SLOT_BYTES = 2 * OP_BYTES;                // A and B of one pair: 64 KB


// Swizzles.  K-major pair tile [256 rows][64 k] (128-byte rows): physical chunk p of
// row r holds logical chunk p ^ ((r >> 1) & 7); a ds_read_b128 is served 16 consecutive
// lanes (16 consecutive rows, one logical chunk) at a time over 64 four-byte banks, and
// rows r, r+1 differ in bit 3 of the bank group while (r >> 1) & 7 spreads the eight
// row pairs, so the 16 reads hit distinct banks.  MN-major tile [32 k][256 cols]
// (512-byte rows): physical chunk p of k-row r holds logical chunk p ^ swz_mn(r).
__device__ __forceinline__ int swz_mn(int r) { return ((r & 3) << 2) ^ (((r >> 3) & 1) << 1); }
// Gate/up sub-tile [32 k][128 cols] (256-byte k rows): physical chunk = logical chunk ^
// swz_split(k row).
__device__ __forceinline__ int swz_split(int r) { return (4 * (r & 3)) ^ (((r >> 3) & 1) << 1); }
// K-major single-k-step tile [256 rows][32 k] (64-byte rows): physical chunk p of row r
// holds logical chunk p ^ swz_k(r).  Chosen by measurement (SQ_LDS_BANK_CONFLICT over
// SQ_LDS_IDX_ACTIVE in the forward passes, whose A operand is the only user): (r >> 1) & 3
// gives 1.3%; (r >> 2) & 3, r & 3 and ((r >> 2) ^ (r >> 4)) & 3 each spend 40% of the
// LDS cycles in bank conflicts.
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 3; }

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

// Byte address of a K-major fragment of a single-k-step tile: row of the tile, chunk.
__device__ __forceinline__ uint32_t addr_k(uint32_t tile, int row, int chunk) {
    return tile + row * 64 + ((chunk ^ swz_k(row)) << 4);
}
// Byte address of the first of the two transpose reads of an MN-major fragment:
// columns [c0, c0+16) of the tile; lane group g = lane/16 reads k rows 8g + [0, 4) and, in
// the second read 4 k rows (2048 bytes) further with the same swizzle, 8g + [4, 8).
__device__ __forceinline__ uint32_t addr_mn(uint32_t tile, int c0, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int col = c0 + 4 * (s & 3);
    const int kr = 8 * g + (s >> 2);
    return tile + kr * 512 + (((col >> 3) ^ swz_mn(kr)) << 4) + (col & 7) * 2;
}

// Gate/up forward B tile: two sub-tiles [32 k][128 cols] (W_g columns, then W_u), 256-byte
// k rows, physical chunk = logical chunk ^ swz_split(k).  A 32-lane half of a transpose
// read covers k rows 8g + [0, 4) for two lane groups g, 32 bytes each, which the swizzle
// spreads over all 64 banks.  The second read of a fragment is 4 k rows (1024 bytes)
// further.
__device__ __forceinline__ uint32_t addr_mn_split(uint32_t sub, int c0, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int col = c0 + 4 * (s & 3);
    const int kr = 8 * g + (s >> 2);
    return sub + kr * 256 + (((col >> 3) ^ swz_split(kr)) << 4) + (col & 7) * 2;
}
__device__ __forceinline__ void ds_tr_pair_1k(s16x4_t& lo, s16x4_t& hi, uint32_t addr) {
    lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr);
    hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(addr + 1024));
}

// Weight-gradient output: written once and not read by this layer again, so it is
// stored nontemporally (it does not displace the operand panels in L2).
__device__ __forceinline__ void store_stream(bf16_t* p, const u32x4& v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (u32x4_t*)p);
}

template <int N> struct Frag {
    s16x4_t lo[N], hi[N];  // MN-major fragments (two transpose reads)
    u32x4_t q[N];          // K-major fragments (one read)
};

template <bool MN, int N>
__device__ __forceinline__ bf16x8_t frag_value(const Frag<N>& f, int i) {
    if (MN) {
        s16x8_t v = __builtin_shufflevector(f.lo[i], f.hi[i], 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8_t, v);
    }
    return __builtin_bit_cast(bf16x8_t, f.q[i]);
}

// Epilogue sigmoid: hardware exp and reciprocal (about 1 ulp each; the results are
// rounded to bf16).  a -> -inf gives rcp(inf) = 0, a -> +inf gives rcp(1) = 1.
__device__ __forceinline__ float fast_sigmoid(float a) {
    return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// PAIRED (the two dgrads): stage pairs of k-steps, so that every direct-load instruction
// reads whole 128-byte lines (a K-major k-step row is only 64 bytes).  With branch-free
// steady-state k-steps in both schemes, pairs ran 2-8% faster than single k-steps on every
// layer shape measured (row pitches 4 to 112 KB), also against the half-height last tiles
// of the short-segment shapes.
template <int MODE, bool PAIRED> struct Traits {
    static constexpr bool a_mn = MODE == GG_WGRAD_DOWN || MODE == GG_WGRAD_GATEUP;
    static constexpr bool b_mn = MODE == GG_FWD_GATEUP || MODE == GG_FWD_DOWN || a_mn;
    static constexpr bool paired = PAIRED;
    static_assert(!PAIRED || MODE == GG_DGRAD_GATEUP || MODE == GG_DGRAD_DOWN,
                  "the dgrads stage pairs");
};

// Buffer resource over the raw byte range [base, base + bytes): a direct load through it
// takes a 32-bit per-lane offset (half the address traffic of a 64-bit flat address), and
// the hardware returns zeros for offsets at or past `bytes`, which the weight-gradient
// passes use for the k rows past the end of a segment.
//
// The direct load (16 bytes per lane; the 64 lanes fill 1 KB of LDS starting at the
// wave-uniform address in M0) is written as inline asm so that the compiler does not
// treat every later LDS read as possibly aliasing it (it would wait for all loads in
// flight before each read); completion is awaited explicitly with s_waitcnt vmcnt
// before the barrier that publishes a stage.  The asm has no register outputs.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc(uint64_t base, uint32_t bytes) {
    i32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));  // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;  // raw buffer, 32-bit data format
    return r;
}
__device__ __forceinline__ void lds_dma16_buf(const i32x4_t& rsrc, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds_addr) : "memory", "m0");
}

// One 256-thread group of four waves computes while the other loads; a SIMD runs one
// wave of each group.  Block barriers alternate the two roles.
constexpr int NTHREADS = 512;

// One output tile of BM_ = 32 RB rows (RB = 8: 256 rows; RB = 4: a half-height tile of
// 128 rows for a segment's last rows) by 256 columns: wave w computes rows
// 16 RB (w & 1) .. +16 RB - 1 and columns 64 (w >> 1) .. +63 as RB x 4 MFMA blocks.  A
// half-height tile keeps the full tile's B operand, LDS layout and schedule; its A tile
// is 128 rows (two direct loads per wave and k-step instead of four) and each compute
// phase has 16 MFMAs.
// s_waitcnt vmcnt(N) for a compile-time N.
template <int N> __device__ __forceinline__ void vm_wait() {
    static_assert(N == 0 || N == 2 || N == 4 || N == 8, "vmcnt values used by the ring");
    if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int MODE, bool PAIRED, int RB>
__device__ __forceinline__ void gg_tile(const GemmArgs& g, uint32_t smem_base, int e, int m0, int m_lim,
                                        int n0, int k_lo, int k_hi, int nk) {
    static_assert(RB == 8 || (RB == 4 && !PAIRED && MODE <= GG_DGRAD_GATEUP),
                  "half-height tiles serve the row passes on the single-k-step ring");
    using TR = Traits<MODE, PAIRED>;
    constexpr int WROWS = 16 * RB;  // output rows of a wave

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wv >> 2;   // waves w and w + 4 share a SIMD and sit in different groups
    const int wq = wv & 3;     // wave within its group
    const int wm = wv & 1;     // output rows wm*WROWS .. +WROWS-1 of the tile
    const int wn = wv >> 1;    // output columns wn*64 .. +63 (gate/up: features wn*32 .. +31)
    const int d = g.d, f = g.f;

    const bf16_t* A0 = (const bf16_t*)g.A0;
    const bf16_t* A1 = (const bf16_t*)g.A1;
    const bf16_t* B0 = (const bf16_t*)g.B0;
    const bf16_t* B1 = (const bf16_t*)g.B1;

    f32x4_t acc[RB][4];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

    // Down dgrad: the SwiGLU backward of the epilogue reads a and b at every output
    // element.  The loads of band 0 are issued before the main loop (they are older than
    // every direct load, so the vmcnt waits of the loop still cover the loads they
    // target), those of band i+1 before band i is processed; rows are clamped to valid
    // rows (a row past the segment is neither used nor stored).
    u32x4 xa[2][4], xb[2][4];
    auto load_x = [&](int i, int buf) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int q = lane + 64 * t;
            const int row = min(m0 + wm * WROWS + i * 32 + (q >> 3), m_lim - 1);
            const int64_t o = (int64_t)row * f + n0 + wn * 64 + (q & 7) * 8;
            xa[buf][t] = *(const u32x4*)((const bf16_t*)g.X0 + o);
            xb[buf][t] = *(const u32x4*)((const bf16_t*)g.X1 + o);
        }
    };
    if constexpr (MODE == GG_DGRAD_DOWN) load_x(0, 0);

    if constexpr (TR::paired) {
        static_assert(MODE == GG_DGRAD_GATEUP || MODE == GG_DGRAD_DOWN, "the paired staging serves the dgrads");
        // ---- direct loads.  K-steps are loaded in pairs (64 k) into two 64 KB slots
        // [A 32 KB | B 32 KB]; group 0 loads A, group 1 loads B, and wave wq of a group issues
        // instructions 8wq .. 8wq+7 of the 32 (1 KB each) that cover one operand of a pair.
        // An operand sits as [256 rows][64 k] with 128-byte rows, so that every instruction
        // reads whole 128-byte lines: instruction ii covers rows 8ii + lane/8, physical chunk
        // lane%8 (swizzle chunk ^ ((row >> 1) & 7)).  Every load goes through a buffer
        // resource whose base moves with the pair (kbase0 + p * kstride; the gate/up dgrad
        // switches to kbase1 at k = f: da with W_g, then db with W_u) and a fixed per-lane
        // byte offset.  Down dgrad: A = d_o rows and B = W_d,e rows n0.., both [.][d].
        const int64_t ld = MODE == GG_DGRAD_DOWN ? d : f;  // row pitch of both operands
        uint64_t kbase0, kbase1;
        if (grp == 0) {
            kbase0 = (uint64_t)(A0 + (int64_t)m0 * ld);
            kbase1 = MODE == GG_DGRAD_DOWN ? kbase0 : (uint64_t)(A1 + (int64_t)m0 * ld);
        } else if (MODE == GG_DGRAD_DOWN) {
            kbase0 = (uint64_t)(B0 + (int64_t)e * f * d + (int64_t)n0 * d);
            kbase1 = kbase0;
        } else {
            kbase0 = (uint64_t)(B0 + (int64_t)e * d * f + (int64_t)n0 * f);
            kbase1 = (uint64_t)(B1 + (int64_t)e * d * f + (int64_t)n0 * f);
        }
        const uint64_t kstride = (uint64_t)KP * 2;
        const int psplit = MODE == GG_DGRAD_DOWN ? 0x7FFFFFFF : f / KP;
        const int np = (nk + 1) >> 1;
        uint32_t voff[8];
    #pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int row = (wq * 8 + u) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ ((row >> 1) & 7);
            // A: rows past the segment read any valid row (their results are not stored)
            const int r = grp == 0 ? min(m0 + row, m_lim - 1) - m0 : row;
            voff[u] = (uint32_t)(((int64_t)r * ld + c * 8) * 2);
        }

        // Issue the u-th of this wave's eight direct loads of pair p.
        auto issue_one = [&](int p, int u) {
            const uint32_t dst = smem_base + (p & 1) * SLOT_BYTES + grp * OP_BYTES + (wq * 8 + u) * 1024;
            const bool second = p >= psplit;
            const uint64_t base = (second ? kbase1 : kbase0) + (uint64_t)(second ? p - psplit : p) * kstride;
            lds_dma16_buf(make_rsrc(base, 0xFFFFFFF0u), voff[u], dst);
        };

        // Per-lane LDS byte offsets (within a slot, for the first k-step of a pair) of this
        // wave's fragment reads: 8 A fragments (16 rows each) and 4 B fragments (16 columns
        // each).  For the second k-step of the pair an offset flips bit 6 (its chunk index is
        // 4 higher and the swizzle only touches the low 3 bits of it).
        auto addr_k64 = [&](uint32_t op, int row, int chunk) -> uint32_t {
            return op + row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
        };
        uint32_t a_rd[8], b_rd[4];
    #pragma unroll
        for (int i = 0; i < 8; ++i) a_rd[i] = addr_k64(0, wm * 128 + i * 16 + (lane & 15), lane >> 4);
    #pragma unroll
        for (int j = 0; j < 4; ++j) b_rd[j] = addr_k64(OP_BYTES, wn * 64 + j * 16 + (lane & 15), lane >> 4);

        Frag<8> fa;
        Frag<4> fb;
        auto read_step = [&](int kt) {
            const uint32_t slot = smem_base + ((kt >> 1) & 1) * SLOT_BYTES;
            const uint32_t hk = (uint32_t)(kt & 1) << 6;  // second k-step of the pair
    #pragma unroll
            for (int i = 0; i < 8; ++i) ds_b128(fa.q[i], slot + (a_rd[i] ^ hk));
    #pragma unroll
            for (int j = 0; j < 4; ++j) ds_b128(fb.q[j], slot + (b_rd[j] ^ hk));
        };


        // Schedule.  Memory phase M(k): read all fragments of k-step k.  Compute phase C(k):
        // the 32 MFMAs of k-step k.  Group 0 runs M(0) C(0) M(1) C(1) ..., group 1 the same
        // one phase later, with a block barrier between phases: while one wave of a SIMD
        // issues MFMAs, the other reads LDS.  Pairs 0 and 1 are loaded up front; pair p+1
        // (p >= 1) goes into the slot of pair p-1 once both groups have read it: group 1
        // issues its eight loads between the MFMAs of C(2p-1), group 0 between those of C(2p).
        // Pair p+1 has landed before the barrier that opens M(2p+2) of group 0: group 0 waits
        // at the end of C(2p+1), group 1 at the end of M(2p+1).  Every wave passes 2 nk + 2
        // barriers.
        if (nk > 0) {
    #pragma unroll
            for (int u = 0; u < 8; ++u) issue_one(0, u);
            if (np > 1) {
    #pragma unroll
                for (int u = 0; u < 8; ++u) issue_one(1, u);
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            if (grp == 1) __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);

            // One k-step.  KIND 0: any k-step, every condition evaluated at run time; KIND 1
            // and 2: the even and odd k-step of a pair p with 1 <= p and p + 2 < np, whose
            // refills (group 0 loads pair p + 1 in the even one, group 1 pair p + 2 in the
            // odd one) and waits are fixed.  G: this wave's group, a compile-time constant
            // (the k-loop runs as one copy per group, so the lean pairs carry no branches).
            auto kstep = [&](int kt, auto kindc, auto grpc) {
                constexpr int KIND = decltype(kindc)::value;
                constexpr int G = decltype(grpc)::value;
                const int g = G < 0 ? grp : G;
                const bool pair_end = KIND == 1 ? false : KIND == 2 ? true
                                    : ((kt & 1) && (kt >> 1) + 1 < np);  // pair kt/2 + 1 due next
                // ---- memory phase
                read_step(kt);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (g == 1 && pair_end) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                // ---- compute phase
                __builtin_amdgcn_s_setprio(1);
                const int pi = KIND == 1 ? (kt >> 1) + 1 : KIND == 2 ? ((kt + 1) >> 1) + 1
                             : g == 0 ? ((kt & 1) == 0 && kt >= 2 ? (kt >> 1) + 1 : np)
                                      : ((kt & 1) ? ((kt + 1) >> 1) + 1 : np);
                const bool refill = KIND == 1 ? g == 0 : KIND == 2 ? g == 1 : pi < np;
    #pragma unroll
                for (int q = 0; q < 32; ++q) {
                    // snake order: consecutive MFMAs differ in one operand only (the
                    // fewest operand changes, which lowers the matrix cores' power)
                    const int i = q >> 2, j = (i & 1) ? 3 - (q & 3) : (q & 3);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        frag_value<TR::b_mn>(fb, j), frag_value<TR::a_mn>(fa, i), acc[i][j], 0, 0, 0);
                    if ((q & 3) == 1 && refill) {
                        __builtin_amdgcn_sched_barrier(0);
                        issue_one(pi, q >> 2);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                __builtin_amdgcn_s_setprio(0);
                if (g == 0 && pair_end) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            };
            using general = std::integral_constant<int, 0>;
            using even = std::integral_constant<int, 1>;
            using odd = std::integral_constant<int, 2>;
            auto kloop = [&](auto gc) {
                int kt = 0;
                for (; kt < min(nk, 2); ++kt) kstep(kt, general{}, gc);
                if (np >= 4) {
                    for (int p = 1; p + 2 < np; ++p) {
                        kstep(2 * p, even{}, gc);
                        kstep(2 * p + 1, odd{}, gc);
                    }
                    kt = 2 * (np - 2);
                }
                for (; kt < nk; ++kt) kstep(kt, general{}, gc);
            };
            if (grp == 0) kloop(std::integral_constant<int, 0>{});
            else kloop(std::integral_constant<int, 1>{});
            if (grp == 0) __builtin_amdgcn_s_barrier();
        }
    } else {
        // ---- this wave's share of the direct loads: group 0 fills the A tile of every
        // stage, group 1 the B tile; wave wq of a group issues instructions 4wq .. 4wq+3 of
        // the 16 that cover one 16 KB operand tile.
        // K-major: instruction ii covers tile rows ii*16 + lane/4, physical chunk lane%4.
        // MN-major: instruction ii covers k rows ii*2 + lane/32, physical chunk lane%32.
        // Gate/up forward B: instruction ii covers k rows 4*(ii%8) + lane/16 of sub-tile ii/8
        // (W_g, then W_u), physical chunk lane%16.
        // Every operand is read through a buffer resource whose base moves with the k-step
        // (kbase0 + kt * kstride; the gate/up dgrad switches to kbase1 at k = f) and a fixed
        // per-lane byte offset.
        const bool mn = grp == 0 ? TR::a_mn : TR::b_mn;
        const int64_t lda = (MODE == GG_FWD_GATEUP || MODE == GG_DGRAD_DOWN) ? d : f;
        // row pitch (elements) of this wave's operand
        const int64_t ld = grp == 0 ? (TR::a_mn ? (MODE == GG_WGRAD_DOWN ? f : d) : lda)
                         : (MODE == GG_DGRAD_DOWN || MODE == GG_FWD_DOWN || MODE == GG_WGRAD_DOWN) ? d : f;
        uint64_t kbase0, kbase1 = 0;
        if (grp == 0) {
            if (TR::a_mn) kbase0 = (uint64_t)(A0 + (int64_t)k_lo * ld);
            else kbase0 = (uint64_t)(A0 + (int64_t)m0 * ld), kbase1 = (uint64_t)(A1 + (int64_t)m0 * ld);
        } else if (MODE == GG_FWD_DOWN) {
            kbase0 = (uint64_t)(B0 + (int64_t)e * f * d);
        } else if (MODE == GG_DGRAD_DOWN) {
            kbase0 = (uint64_t)(B0 + (int64_t)e * f * d + (int64_t)n0 * d);
        } else if (MODE == GG_DGRAD_GATEUP) {
            kbase0 = (uint64_t)(B0 + (int64_t)e * d * f + (int64_t)n0 * f);
            kbase1 = (uint64_t)(B1 + (int64_t)e * d * f + (int64_t)n0 * f);
        } else if (MODE == GG_WGRAD_DOWN) {
            kbase0 = (uint64_t)(B0 + (int64_t)k_lo * d);
        } else if (MODE == GG_WGRAD_GATEUP) {
            kbase0 = (uint64_t)((n0 < f ? B0 : B1) + (int64_t)k_lo * f);
        } else {  // gate/up forward B: waves 0-1 of the group load W_g, waves 2-3 W_u
            kbase0 = (uint64_t)((wq >= 2 ? B1 : B0) + (int64_t)e * d * f + n0);
        }
        const uint64_t kstride = mn ? (uint64_t)BK * ld * 2 : (uint64_t)BK * 2;
        const int ksplit = MODE == GG_DGRAD_GATEUP ? f / BK : nk;
        // direct loads per wave and k-step: the A tile has 16 RB rows (RB / 2 loads of 16
        // rows per wave of group 0), the B tile 256 (four per wave of group 1)
        constexpr int LA = RB / 2;
        const int nl = grp == 0 ? LA : 4;
        uint32_t voff[4];
    #pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ii = wq * (grp == 0 ? LA : 4) + u;
            if (MODE == GG_FWD_GATEUP && grp == 1) {
                const int kr = 4 * (ii & 7) + (lane >> 4);
                const int c = (lane & 15) ^ swz_split(kr);
                voff[u] = (uint32_t)(((int64_t)kr * f + c * 8) * 2);
            } else if (!mn) {
                const int row = ii * 16 + (lane >> 2);
                const int c = (lane & 3) ^ swz_k(row);
                // A: rows past the segment read any valid row (their results are not stored)
                const int r = grp == 0 ? min(m0 + row, m_lim - 1) - m0 : row;
                voff[u] = (uint32_t)(((int64_t)r * ld + c * 8) * 2);
            } else {
                const int kr = ii * 2 + (lane >> 5);
                const int c = (lane & 31) ^ swz_mn(kr);
                const int col0 = grp == 0 ? m0 : (MODE == GG_WGRAD_GATEUP && n0 >= f ? n0 - f : n0);
                voff[u] = (uint32_t)(((int64_t)kr * ld + col0 + c * 8) * 2);
            }
        }

        // Issue the u-th of this wave's nl direct loads of k-step kt into stage st.
        auto issue_one = [&](int kt, int st, int u) {
            const uint32_t dst = smem_base + st * STEP_STAGE_BYTES + grp * STEP_TILE_BYTES + (wq * nl + u) * 1024;
            {
                const bool second = kt >= ksplit;
                const uint64_t base = (second ? kbase1 : kbase0) +
                                      (uint64_t)(second ? kt - ksplit : kt) * kstride;
                uint32_t bytes = 0xFFFFFFF0u;
                if (TR::a_mn) {
                    // weight gradients: k rows past the segment read as zeros
                    const int64_t rows_left = (int64_t)(k_hi - k_lo) - (int64_t)kt * BK;
                    const int64_t nb = rows_left * ld * 2;
                    bytes = nb >= (int64_t)0xFFFFFFF0 ? 0xFFFFFFF0u : (uint32_t)nb;
                }
                lds_dma16_buf(make_rsrc(base, bytes), voff[u], dst);
            }
        };
        auto issue = [&](int kt, int st) {
    #pragma unroll
            for (int u = 0; u < 4; ++u)
                if (u < nl) issue_one(kt, st, u);
        };

        // Per-lane LDS byte offsets (within a stage) of this wave's fragment reads:
        // RB A fragments (16 rows each) and 4 B fragments (16 columns each).
        uint32_t a_rd[RB], b_rd[4];
    #pragma unroll
        for (int i = 0; i < RB; ++i)
            a_rd[i] = TR::a_mn ? addr_mn(0, wm * WROWS + i * 16, lane)
                               : addr_k(0, wm * WROWS + i * 16 + (lane & 15), lane >> 4);
    #pragma unroll
        for (int j = 0; j < 4; ++j) {
            // gate/up: j = 0, 1 read the W_g sub-tile, j = 2, 3 the W_u sub-tile
            const int c0 = wn * 64 + j * 16;
            b_rd[j] = MODE == GG_FWD_GATEUP ? addr_mn_split(STEP_TILE_BYTES + (j >> 1) * 8192, wn * 32 + (j & 1) * 16, lane)
                    : TR::b_mn ? addr_mn(STEP_TILE_BYTES, c0, lane)
                               : addr_k(STEP_TILE_BYTES, c0 + (lane & 15), lane >> 4);
        }

        Frag<RB> fa;
        Frag<4> fb;
        auto read_stage = [&](uint32_t stage) {
    #pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (TR::a_mn) ds_tr_pair(fa.lo[i], fa.hi[i], stage + a_rd[i]);
                else ds_b128(fa.q[i], stage + a_rd[i]);
            }
    #pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (MODE == GG_FWD_GATEUP) ds_tr_pair_1k(fb.lo[j], fb.hi[j], stage + b_rd[j]);
                else if (TR::b_mn) ds_tr_pair(fb.lo[j], fb.hi[j], stage + b_rd[j]);
                else ds_b128(fb.q[j], stage + b_rd[j]);
            }
        };


        // Wait until the `pending` newest of this wave's loads at most are in flight (nl per
        // k-step).
        auto wait_loads = [&](int pending_ksteps) {
            if (RB == 8 || nl == 4) {
                if (pending_ksteps >= 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                else if (pending_ksteps == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            } else {
                if (pending_ksteps >= 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                else if (pending_ksteps == 1) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
        };

        // Schedule.  Memory phase M(k): read all fragments of k-step k.  Compute phase C(k):
        // the 32 MFMAs of k-step k, with this wave's four loads of k-step k+3 (into the stage
        // k-step k-1 used, which both groups have read by then) between them.  Group 0 runs
        // M(0) C(0) M(1) C(1) ..., group 1 the same one phase later, with a block barrier
        // between phases: while one wave of a SIMD issues MFMAs, the other reads LDS.
        // Before the barrier that opens M(k+1) of group 0, each wave has waited for its own
        // loads of k-step k+1: group 0 at the end of C(k) (k-steps k+2, k+3 may be in
        // flight), group 1 at the end of M(k) (k+2 may be).  Every wave passes 2 nk + 2
        // barriers.
        if (nk > 0) {
            issue(0, 0);
            if (nk > 1) issue(1, 1);
            if (nk > 2) issue(2, 2);
            wait_loads(min(nk, 3) - 1);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            if (grp == 1) __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);

            // LEAN: a k-step whose refill target kt + 3 exists (kt + 3 < nk); its waits are
            // then fixed and its loads unconditional, so the steady state has no branches.
            // G: this wave's group when the k-loop runs as one copy per group (the forward
            // passes: 1-2% faster that way, the weight gradients 1-3% slower), else -1.
            auto kstep = [&](int kt, auto lean, auto gc) {
                constexpr bool LEAN = decltype(lean)::value;
                constexpr int G = decltype(gc)::value;
                const int g = G < 0 ? grp : G;
                // wait until at most `pending` k-steps of this wave's loads are in flight
                auto wait_pending = [&](int pending) {
                    if constexpr (G < 0) {
                        wait_loads(pending);
                    } else {
                        constexpr int NL = G == 0 ? LA : 4;  // this group's loads per k-step
                        if (pending >= 2) vm_wait<2 * NL>();
                        else if (pending == 1) vm_wait<NL>();
                        else vm_wait<0>();
                    }
                };
                // ---- memory phase
                read_stage(smem_base + (kt & (STEP_STAGES - 1)) * STEP_STAGE_BYTES);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (g == 1) {
                    // this wave's loads of k-step kt + 1 have landed (kt + 2 may be in flight)
                    if (LEAN) wait_pending(1);
                    else if (kt + 1 < nk) wait_pending(min(1, nk - 2 - kt));
                }
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                // ---- compute phase
                __builtin_amdgcn_s_setprio(1);
                const bool refill = LEAN || kt + 3 < nk;
                const int st3 = (kt + 3) & (STEP_STAGES - 1);
    #pragma unroll
                for (int q = 0; q < 4 * RB; ++q) {
                    // snake order: consecutive MFMAs differ in one operand only (the
                    // fewest operand changes, which lowers the matrix cores' power)
                    const int i = q >> 2, j = (i & 1) ? 3 - (q & 3) : (q & 3);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        frag_value<TR::b_mn>(fb, j), frag_value<TR::a_mn>(fa, i), acc[i][j], 0, 0, 0);
                    // the wave's loads spread over the phase: every 8 MFMAs, or every 4 for
                    // the four B loads of a half-height tile's 16 MFMAs
                    if (RB == 8 || g == 0) {
                        if ((q & 7) == 2 && refill) {
                            __builtin_amdgcn_sched_barrier(0);
                            issue_one(kt + 3, st3, q >> 3);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    } else {
                        if ((q & 3) == 2 && refill) {
                            __builtin_amdgcn_sched_barrier(0);
                            issue_one(kt + 3, st3, q >> 2);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
                __builtin_amdgcn_s_setprio(0);
                if (g == 0) {
                    // this wave's loads of k-step kt + 1 have landed (kt + 2, kt + 3 may be
                    // in flight)
                    if (LEAN) wait_pending(2);
                    else if (kt + 1 < nk) wait_pending(min(2, nk - 2 - kt));
                }
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            };
            auto kloop = [&](auto gc) {
                int kt = 0;
                for (; kt + 3 < nk; ++kt) kstep(kt, std::integral_constant<bool, true>{}, gc);
                for (; kt < nk; ++kt) kstep(kt, std::integral_constant<bool, false>{}, gc);
            };
            if constexpr (MODE == GG_FWD_GATEUP || MODE == GG_FWD_DOWN) {
                if (grp == 0) kloop(std::integral_constant<int, 0>{});
                else kloop(std::integral_constant<int, 1>{});
            } else {
                kloop(std::integral_constant<int, -1>{});
            }
            if (grp == 0) __builtin_amdgcn_s_barrier();
        }
    }

    // Epilogue.  The MFMAs take the B fragment as their first operand, so each 16x16
    // block accumulates C transposed: lane holds row (lane & 15) of the block and the
    // four consecutive columns 4*(lane/16) + r, r = 0..3 (one 16-byte LDS write).  Each
    // wave stages one 32-row band of its results (32 x 64; fp32, or bf16 for the weight
    // gradients) at a time in a private 8.5 KB of LDS, then every lane handles 8-column
    // chunks: 16-byte loads of epilogue inputs and 16-byte stores.  Every wave has passed
    // the last barrier after the last reads of the operand stages, and no direct load is
    // in flight.
    typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
    constexpr int P = 68;  // band row pitch in floats
    const uint32_t wbase = smem_base + wv * (32 * P * 4);
    const int cl = lane & 15;
    const int cq = 4 * (lane >> 4);
    if constexpr (MODE == GG_WGRAD_DOWN || MODE == GG_WGRAD_GATEUP) {
        // The weight gradients store bf16(acc) and nothing else, so the accumulators are
        // rounded before staging: half the LDS bytes of the fp32 band (one 8-byte write per
        // 16x16 block and lane, one 16-byte read per 8-column chunk).  No MFMA overlaps
        // this epilogue, so its LDS time is part of the pass.
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
        // band row pitch in bf16 elements; measured against 80 and 136 (bank conflicts
        // 10.0%, 22.9%, 12.9% of the LDS cycles)
        constexpr int PB = 72;
        const uint32_t bbase = smem_base + wv * (32 * PB * 2);
#pragma unroll
        for (int i = 0; i < RB / 2; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4_t& a4 = acc[2 * i + h][j];
                    const u32x2_t v = {pack_bf16x2(a4[0], a4[1]), pack_bf16x2(a4[2], a4[3])};
                    *(lds_u32x2*)(uintptr_t)(bbase + ((16 * h + cl) * PB + 16 * j + cq) * 2) = v;
                }
            const int row_base = wm * WROWS + i * 32;  // within the block tile
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int q = lane + 64 * t;
                const int rl = q >> 3, cc = q & 7;
                const u32x4_t w = *(const lds_u32x4*)(uintptr_t)(bbase + (rl * PB + cc * 8) * 2);
                const u32x4 v = {w[0], w[1], w[2], w[3]};
                const int rt = row_base + rl;     // row within the block tile
                const int ct = wn * 64 + cc * 8;  // column within the block tile
                if (MODE == GG_WGRAD_DOWN) {
                    const int64_t o = (int64_t)e * f * d + (int64_t)(m0 + rt) * d + n0 + ct;
                    store_stream((bf16_t*)g.C0 + o, v);
                } else {
                    const bool first = n0 < f;
                    bf16_t* out = (bf16_t*)(first ? g.C0 : g.C1);
                    const int64_t o = (int64_t)e * d * f + (int64_t)(m0 + rt) * f +
                                      (first ? n0 : n0 - f) + ct;
                    store_stream(out + o, v);
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < RB / 2; ++i) {
        if constexpr (MODE == GG_DGRAD_DOWN) {
            if (i + 1 < RB / 2) load_x(i + 1, (i + 1) & 1);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // block row 2i + h: band row 16h + cl, columns 16j + cq .. +3: one 16-byte write
                const f32x4_t& a4 = acc[2 * i + h][j];
                const u32x4_t v = {__float_as_uint(a4[0]), __float_as_uint(a4[1]),
                                   __float_as_uint(a4[2]), __float_as_uint(a4[3])};
                *(lds_u32x4*)(uintptr_t)(wbase + ((16 * h + cl) * P + 16 * j + cq) * 4) = v;
            }
        const int row_base = wm * WROWS + i * 32;  // within the block tile
        if (MODE == GG_FWD_GATEUP) {
            // band columns 0..31: a of features wn*32 + 0..31; columns 32..63: b of the same
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int q = lane + 64 * t;
                const int rl = q >> 2, cc = q & 3;
                const int row = m0 + row_base + rl;
                const uint32_t la = wbase + (rl * P + cc * 8) * 4;
                const uint32_t lb = la + 32 * 4;
                u32x4_t a0 = *(const lds_u32x4*)(uintptr_t)la;
                u32x4_t a1 = *(const lds_u32x4*)(uintptr_t)(la + 16);
                u32x4_t b0 = *(const lds_u32x4*)(uintptr_t)lb;
                u32x4_t b1 = *(const lds_u32x4*)(uintptr_t)(lb + 16);
                if (row < m_lim) {
                    float av[8], bv[8], hv[8];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        av[u] = __uint_as_float(a0[u]); av[u + 4] = __uint_as_float(a1[u]);
                        bv[u] = __uint_as_float(b0[u]); bv[u + 4] = __uint_as_float(b1[u]);
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) hv[u] = av[u] * fast_sigmoid(av[u]) * bv[u];
                    const int64_t o = (int64_t)row * f + n0 + wn * 32 + cc * 8;
                    *(u32x4*)((bf16_t*)g.C0 + o) = Vec16<bf16_t>::pack(av);
                    *(u32x4*)((bf16_t*)g.C1 + o) = Vec16<bf16_t>::pack(bv);
                    *(u32x4*)((bf16_t*)g.C2 + o) = Vec16<bf16_t>::pack(hv);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int q = lane + 64 * t;
                const int rl = q >> 3, cc = q & 7;
                const uint32_t la = wbase + (rl * P + cc * 8) * 4;
                u32x4_t v0 = *(const lds_u32x4*)(uintptr_t)la;
                u32x4_t v1 = *(const lds_u32x4*)(uintptr_t)(la + 16);
                float v[8];
#pragma unroll
                for (int u = 0; u < 4; ++u) { v[u] = __uint_as_float(v0[u]); v[u + 4] = __uint_as_float(v1[u]); }
                const int rt = row_base + rl;              // row within the block tile
                const int ct = wn * 64 + cc * 8;           // column within the block tile
                if (MODE == GG_FWD_DOWN || MODE == GG_DGRAD_GATEUP) {
                    const int row = m0 + rt;
                    const int64_t o = (int64_t)row * d + n0 + ct;
                    if (row < m_lim) {
                        if (g.out_f32) {
                            *(u32x4_t*)((float*)g.C0 + o) = v0;
                            *(u32x4_t*)((float*)g.C0 + o + 4) = v1;
                        } else {
                            *(u32x4*)((bf16_t*)g.C0 + o) = Vec16<bf16_t>::pack(v);
                        }
                    }
                } else if (MODE == GG_DGRAD_DOWN) {
                    const int row = m0 + rt;
                    if (row < m_lim) {
                        const int64_t o = (int64_t)row * f + n0 + ct;
                        float av[8], bv[8], dav[8], dbv[8];
                        Vec16<bf16_t>::unpack(xa[i & 1][t], av);
                        Vec16<bf16_t>::unpack(xb[i & 1][t], bv);
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const float sg = fast_sigmoid(av[u]);
                            dav[u] = v[u] * bv[u] * sg * (1.0f + av[u] * (1.0f - sg));
                            dbv[u] = v[u] * av[u] * sg;
                        }
                        *(u32x4*)((bf16_t*)g.C0 + o) = Vec16<bf16_t>::pack(dav);
                        *(u32x4*)((bf16_t*)g.C1 + o) = Vec16<bf16_t>::pack(dbv);
                    }
                }
                // (the weight gradients returned from their bf16 staging above)
            }
        }
    }
}

// Row passes (MODE <= GG_DGRAD_GATEUP) find their tile from the segment offsets; with HALF,
// a segment whose last row tile holds at most 128 rows runs that tile at half height (the
// tile count is the same).  Weight gradients take tiles::wgrad_tile.
template <int MODE, bool PAIRED, bool HALF>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(2, 2)))
gg_mfma_kernel(GemmArgs g) {
    static_assert(!HALF || (!PAIRED && MODE <= GG_DGRAD_GATEUP), "half tiles: ring row passes");
    __shared__ __attribute__((aligned(1024))) char smem[2 * SLOT_BYTES];
    const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
    const int d = g.d, f = g.f;
    int e = 0, m0 = 0, m_lim = 0, n0 = 0, k_lo = 0, k_hi = 0, nk = 0;
    bool half = false;
    if (MODE <= GG_DGRAD_GATEUP) {
        const int n_tiles = tiles::row_n_tiles(MODE, d, f);
        int nt, mh;
        if (!tiles::row_tile(blockIdx.x, g.offsets, g.E, n_tiles, HALF, g.row_map, e, m0, m_lim,
                             nt, mh))
            return;
        half = mh < BM;
        n0 = nt * (MODE == GG_FWD_GATEUP ? 128 : BN);
        const int K = MODE == GG_FWD_GATEUP ? d : MODE == GG_FWD_DOWN ? f
                    : MODE == GG_DGRAD_DOWN ? d : 2 * f;
        nk = K / BK;
    } else {
        // Weight gradients: a tile's K is its expert's segment (tiles::wgrad_tile gives
        // every XCD the same contiguous share of each expert's tiles).
        int MT, NTl, mi, ni;
        tiles::wgrad_dims(MODE, d, f, MT, NTl);
        if (!tiles::wgrad_tile(blockIdx.x, g.E, MT, NTl, e, mi, ni)) return;
        m0 = mi * BM;
        n0 = ni * BN;
        k_lo = g.offsets[e];
        k_hi = g.offsets[e + 1];
        nk = (k_hi - k_lo + BK - 1) / BK;
    }
    if constexpr (HALF) {
        if (half) {
            gg_tile<MODE, PAIRED, 4>(g, smem_base, e, m0, m_lim, n0, k_lo, k_hi, nk);
            return;
        }
    }
    gg_tile<MODE, PAIRED, 8>(g, smem_base, e, m0, m_lim, n0, k_lo, k_hi, nk);
}

// Weight gradients with short segments, persistent.  One block per CU walks the tiles that
// tiles::wgrad_tile gives its XCD, in the same order as a one-tile-per-block launch, and
// keeps the operand ring running across tile boundaries: during the last three compute
// phases of a tile (when it has at least three k-steps) the refills fetch the next
// tile's first three k-steps, so that tile starts on data already in LDS, and the
// epilogue's stores (128 KB per tile) drain while it runs instead of ahead of its first
// loads.  The stage index runs on over tiles (k-step j of a tile whose first k-step is
// the block's g0-th sits in stage (g0 + j) % 4); the epilogue stages its results in the
// one stage no load targets at that moment, 32 rows per wave at a time.
//
// Waits.  vmcnt counts loads and stores together and retires them in order.  When a
// tile's first k-steps were issued by the previous tile, the previous epilogue's 16
// stores per wave sit between them and the tile's own later loads, so the waits for
// those k-steps (k-steps 0..2) allow the stores to stay in flight; every other wait
// counts exactly the loads issued after the one it waits for.
constexpr int WG_STORES = 16;  // global stores per wave in a weight-gradient epilogue

__device__ __forceinline__ void wait_vm(int n) {
    // n: loads and stores allowed to stay in flight (a multiple of 4, at most 28)
    switch (n) {
        case 28: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
        case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
        case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
        case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// Experts a persistent weight-gradient launch can take (the library's limit on E).
constexpr int WG_MAX_E = 64;

struct WgTile {
    int e, m0, n0, k_lo, nrows, nk;
    bool ok;
};

template <int MODE>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(2, 2)))
gg_wgrad_kernel(GemmArgs g) {
    static_assert(MODE == GG_WGRAD_DOWN || MODE == GG_WGRAD_GATEUP, "weight gradients");
    __shared__ __attribute__((aligned(1024))) char smem[2 * SLOT_BYTES];
    const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_void*)smem;
    const int d = g.d, f = g.f;
    int MT, NTl;
    tiles::wgrad_dims(MODE, d, f, MT, NTl);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wv >> 2;   // group 0 loads A (rows m of dW), group 1 loads B (columns n)
    const int wq = wv & 3;
    const int wm = wv & 1;
    const int wn = wv >> 1;
    const bf16_t* A0 = (const bf16_t*)g.A0;
    const bf16_t* B0 = (const bf16_t*)g.B0;
    const bf16_t* B1 = (const bf16_t*)g.B1;
    // row pitch of this wave's operand: A = h ([rows][f]) or xp ([rows][d]); B = d_o
    // ([rows][d]) or da, db ([rows][f])
    const int64_t ld = grp == 0 ? (MODE == GG_WGRAD_DOWN ? f : d) : (MODE == GG_WGRAD_DOWN ? d : f);
    const uint64_t kstride = (uint64_t)BK * ld * 2;
    // per-lane byte offsets of this wave's four direct loads (MN-major: instruction ii
    // covers k rows 2 ii + lane / 32, physical chunk lane % 32), without the tile's column
    uint32_t vbase[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int ii = wq * 4 + u;
        const int kr = ii * 2 + (lane >> 5);
        const int c = (lane & 31) ^ swz_mn(kr);
        vbase[u] = (uint32_t)(((int64_t)kr * ld + c * 8) * 2);
    }
    uint32_t a_rd[8], b_rd[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) a_rd[i] = addr_mn(0, wm * 128 + i * 16, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) b_rd[j] = addr_mn(STEP_TILE_BYTES, wn * 64 + j * 16, lane);

    // The segment offsets (E + 1 <= WG_MAX_E + 1 values) are staged in LDS once, so that
    // a tile's decode reads them with LDS loads: a vector load at a tile boundary would
    // be followed by a wait for every vector memory operation in flight (the previous
    // epilogue's stores and the prefetched k-steps included), and a scalar load there
    // measured 0.4 µs of latency under this kernel's memory traffic.
    __shared__ int32_t offs_lds[WG_MAX_E + 1];
    if (tid <= g.E) offs_lds[tid] = g.offsets[tid];
    __syncthreads();
    auto decode = [&](int64_t b) {
        WgTile t{0, 0, 0, 0, 0, 0, false};
        int e, mi, ni;
        if (b > 0x7FFFFFFF || !tiles::wgrad_tile((int)b, g.E, MT, NTl, e, mi, ni)) return t;
        e = __builtin_amdgcn_readfirstlane(e);
        t.ok = true;
        t.e = e;
        t.m0 = __builtin_amdgcn_readfirstlane(mi) * BM;
        t.n0 = __builtin_amdgcn_readfirstlane(ni) * BN;
        t.k_lo = __builtin_amdgcn_readfirstlane(offs_lds[e]);
        t.nrows = __builtin_amdgcn_readfirstlane(offs_lds[e + 1]) - t.k_lo;
        t.nk = (t.nrows + BK - 1) / BK;
        return t;
    };
    // this wave's operand of tile t: base at the segment's first row, and the column
    auto src_base = [&](const WgTile& t) -> uint64_t {
        if (grp == 0) return (uint64_t)(A0 + (int64_t)t.k_lo * ld);
        if (MODE == GG_WGRAD_DOWN) return (uint64_t)(B0 + (int64_t)t.k_lo * d);
        return (uint64_t)((t.n0 < f ? B0 : B1) + (int64_t)t.k_lo * f);
    };
    auto src_col = [&](const WgTile& t) -> int {
        return grp == 0 ? t.m0 : (MODE == GG_WGRAD_GATEUP && t.n0 >= f ? t.n0 - f : t.n0);
    };
    // load u of k-step kt of a tile into stage st; k rows past the segment read as zeros
    auto issue_one = [&](const WgTile& t, uint64_t base, int col, int kt, int st, int u) {
        const uint32_t dst = smem_base + st * STEP_STAGE_BYTES + grp * STEP_TILE_BYTES + (wq * 4 + u) * 1024;
        const int64_t nb = ((int64_t)t.nrows - (int64_t)kt * BK) * ld * 2;
        const uint32_t bytes = nb >= (int64_t)0xFFFFFFF0 ? 0xFFFFFFF0u : (uint32_t)nb;
        lds_dma16_buf(make_rsrc(base + (uint64_t)kt * kstride, bytes), vbase[u] + (uint32_t)col * 2, dst);
    };

    Frag<8> fa;
    Frag<4> fb;
    auto read_stage = [&](uint32_t stage) {
#pragma unroll
        for (int i = 0; i < 8; ++i) ds_tr_pair(fa.lo[i], fa.hi[i], stage + a_rd[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) ds_tr_pair(fb.lo[j], fb.hi[j], stage + b_rd[j]);
    };

    int64_t b = blockIdx.x;
    WgTile cur = decode(b);
    int g0 = 0;   // the block's k-steps before this tile (stage of k-step j: (g0 + j) & 3)
    int pre = 0;  // this tile's k-steps issued by the previous tile (0, or min(3, nk))
    while (cur.ok) {
        const WgTile nxt = decode(b + gridDim.x);
        const int nk = cur.nk;
        const bool pf = nk >= 3 && nxt.ok && nxt.nk > 0;
        const uint64_t cbase = src_base(cur);
        const int ccol = src_col(cur);
        const uint64_t nbase = pf ? src_base(nxt) : 0;
        const int ncol = pf ? src_col(nxt) : 0;
        // targets j >= 0 of this tile's load sequence: own k-step j, or the next tile's
        // k-step j - nk (issued during compute phase j - 3)
        auto issued = [&](int j) -> int { return (j < nk || (pf && j - nk < nxt.nk)) ? 1 : 0; };
        auto issue_target = [&](int j, int u) {
            const int st = (g0 + j) & (STEP_STAGES - 1);
            if (j < nk) issue_one(cur, cbase, ccol, j, st, u);
            else issue_one(nxt, nbase, ncol, j - nk, st, u);
        };
        // stores of the previous epilogue still allowed in flight when waiting for k-step j
        auto held = [&](int j) -> int { return (pre > 0 && j <= 2) ? WG_STORES : 0; };

        f32x4_t acc[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

        if (nk > 0) {
            const int n3 = min(nk, 3);
            if (pre == 0) {
                for (int j = 0; j < n3; ++j) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) issue_target(j, u);
                }
            }
            wait_vm(4 * (n3 - 1) + held(0));
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            if (grp == 1) __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);

            // the compute phase of k-step kt loads target kt + 3: its source, column and the
            // bytes left in its segment are carried from phase to phase
            const int64_t kbytes = (int64_t)BK * ld * 2;
            bool tvalid;
            uint64_t tbase;
            int64_t tnb;
            uint32_t tcol2;
            if (3 < nk) {
                tvalid = true;
                tbase = cbase + 3 * kstride;
                tnb = ((int64_t)cur.nrows - 3 * BK) * ld * 2;
                tcol2 = (uint32_t)ccol * 2;
            } else {
                tvalid = pf && 3 - nk < nxt.nk;
                tbase = nbase + (uint64_t)(3 - nk) * kstride;
                tnb = ((int64_t)nxt.nrows - (int64_t)(3 - nk) * BK) * ld * 2;
                tcol2 = (uint32_t)ncol * 2;
            }
            // One k-step: memory phase, then compute phase.  LEAN: a k-step whose target
            // kt + 3 and next target kt + 4 both lie in this tile and which no store of the
            // previous epilogue precedes (2 <= kt, kt + 4 < nk): the waits and the refill
            // are then fixed, and the steady state carries no branches beyond the one-tile
            // kernel's.
            auto kstep = [&](int kt, auto lean) {
                constexpr bool LEAN = decltype(lean)::value;
                // ---- memory phase
                read_stage(smem_base + ((g0 + kt) & (STEP_STAGES - 1)) * STEP_STAGE_BYTES);
                const bool refill = LEAN || tvalid;
                const uint64_t rbase = tbase;
                const uint32_t rbytes = tnb >= (int64_t)0xFFFFFFF0 ? 0xFFFFFFF0u : (uint32_t)tnb;
                const uint32_t rcol2 = tcol2;
                const uint32_t rdst = smem_base + ((g0 + kt + 3) & (STEP_STAGES - 1)) * STEP_STAGE_BYTES +
                                      grp * STEP_TILE_BYTES + wq * 4 * 1024;
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (grp == 1 && (LEAN || kt + 1 < nk)) {
                    if (LEAN || (kt >= 2 && kt + 2 < nk)) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                    else wait_vm(4 * issued(kt + 2) + held(kt + 1));
                }
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                // ---- compute phase, with this wave's four loads of target kt + 3
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int q = 0; q < 32; ++q) {
                    const int i = q >> 2, j = (i & 1) ? 3 - (q & 3) : (q & 3);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        frag_value<true>(fb, j), frag_value<true>(fa, i), acc[i][j], 0, 0, 0);
                    if ((q & 7) == 2 && refill) {
                        __builtin_amdgcn_sched_barrier(0);
                        lds_dma16_buf(make_rsrc(rbase, rbytes), vbase[q >> 3] + rcol2, rdst + (q >> 3) * 1024);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                __builtin_amdgcn_s_setprio(0);
                // the next target, kt + 4: this tile's k-step, or the next tile's
                if (LEAN || kt + 4 < nk) {
                    tbase += kstride;
                    tnb -= kbytes;
                } else if (kt + 4 == nk) {
                    tvalid = pf;
                    tbase = nbase;
                    tnb = (int64_t)nxt.nrows * ld * 2;
                    tcol2 = (uint32_t)ncol * 2;
                } else {
                    tvalid = tvalid && kt + 4 - nk < nxt.nk;
                    tbase += kstride;
                    tnb -= kbytes;
                }
                if (grp == 0 && (LEAN || kt + 1 < nk)) {
                    if (LEAN || (kt >= 2 && kt + 3 < nk)) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                    else wait_vm(4 * (issued(kt + 2) + issued(kt + 3)) + held(kt + 1));
                }
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            };
            using lean = std::integral_constant<bool, true>;
            using general = std::integral_constant<bool, false>;
            const int head = min(nk, 2);
            int kt = 0;
            for (; kt < head; ++kt) kstep(kt, general{});
            for (; kt + 4 < nk; ++kt) kstep(kt, lean{});
            for (; kt < nk; ++kt) kstep(kt, general{});
            if (grp == 0) __builtin_amdgcn_s_barrier();
        }

        // ---- epilogue: bf16(acc), staged 32 rows at a time in the stage no load targets
        // (the one after the next tile's prefetched k-steps; 4 KB per wave, rows of 128
        // bytes whose 16-byte chunks are XOR-swizzled by row), then 16-byte streaming stores.
        {
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
            typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
            const uint32_t bbase = smem_base + ((g0 + nk + 3) & (STEP_STAGES - 1)) * STEP_STAGE_BYTES +
                                   wv * (32 * 128);
            const int cl = lane & 15;
            const int cq = 4 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f32x4_t& a4 = acc[2 * i + h][j];
                        const u32x2_t v = {pack_bf16x2(a4[0], a4[1]), pack_bf16x2(a4[2], a4[3])};
                        const int row = 16 * h + cl, col = 16 * j + cq;  // col: 4 bf16, half a chunk
                        *(lds_u32x2*)(uintptr_t)(bbase + row * 128 + (((col >> 3) ^ (row & 7)) << 4) + (col & 7) * 2) = v;
                    }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int q = lane + 64 * t;
                    const int rl = q >> 3, cc = q & 7;
                    const u32x4_t w = *(const lds_u32x4*)(uintptr_t)(bbase + rl * 128 + ((cc ^ (rl & 7)) << 4));
                    const u32x4 v = {w[0], w[1], w[2], w[3]};
                    const int rt = wm * 128 + i * 32 + rl;  // row within the tile
                    const int ct = wn * 64 + cc * 8;        // column within the tile
                    if (MODE == GG_WGRAD_DOWN) {
                        const int64_t o = (int64_t)cur.e * f * d + (int64_t)(cur.m0 + rt) * d + cur.n0 + ct;
                        store_stream((bf16_t*)g.C0 + o, v);
                    } else {
                        const bool first = cur.n0 < f;
                        bf16_t* out = (bf16_t*)(first ? g.C0 : g.C1);
                        const int64_t o = (int64_t)cur.e * d * f + (int64_t)(cur.m0 + rt) * f +
                                          (first ? cur.n0 : cur.n0 - f) + ct;
                        store_stream(out + o, v);
                    }
                }
            }
        }
        pre = pf ? min(3, nxt.nk) : 0;
        g0 += nk;
        cur = nxt;
        b += gridDim.x;
    }
}

template <int MODE, bool PAIRED = false, bool HALF = false>
hipError_t launch_mode(const GemmArgs& a, unsigned g8, hipStream_t s) {
    gg_mfma_kernel<MODE, PAIRED, HALF><<<g8, NTHREADS, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

bool mfma_shape_ok(const moe_desc& d) {
    return d.dtype == MOE_BF16 && d.d % 256 == 0 && d.f % 256 == 0 && d.d > 0 && d.f > 0;
}

hipError_t launch_gemm_mfma(GemmMode mode, const GemmArgs& args, hipStream_t s) {
    GemmArgs a = args;
    a.row_map = tiles::row_map(mode, a.R, a.E);
    const int64_t g8 = tiles::grid_blocks(mode, a.E, a.R, a.d, a.f);
    if (g8 <= 0) return hipSuccess;
    if (g8 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const unsigned G = (unsigned)g8;
    // Short segments (at most 640 rows per expert by the buffer bound) leave many experts
    // a last row tile of at most 128 rows: the forward passes then take the kernel that
    // runs such a tile at half height, and the weight gradients (whose tiles then have few
    // k-steps) the persistent kernel.  Longer segments keep the one-tile-per-block kernels.
    // The dgrads stage pairs of k-steps on every shape (full-height tiles).
    const bool half = (int64_t)a.R <= 640LL * a.E;
    switch (mode) {
        case GG_FWD_GATEUP:
            return half ? launch_mode<GG_FWD_GATEUP, false, true>(a, G, s)
                        : launch_mode<GG_FWD_GATEUP>(a, G, s);
        case GG_FWD_DOWN:
            return half ? launch_mode<GG_FWD_DOWN, false, true>(a, G, s)
                        : launch_mode<GG_FWD_DOWN>(a, G, s);
        case GG_DGRAD_DOWN:
            return launch_mode<GG_DGRAD_DOWN, true>(a, G, s);
        case GG_DGRAD_GATEUP:
            return launch_mode<GG_DGRAD_GATEUP, true>(a, G, s);
        case GG_WGRAD_DOWN:
        default: {
            if (!half) {
                return mode == GG_WGRAD_DOWN ? launch_mode<GG_WGRAD_DOWN>(a, G, s)
                                             : launch_mode<GG_WGRAD_GATEUP>(a, G, s);
            }
            // short segments (few k-steps per tile): one persistent block per CU (at most
            // one fits: 128 KB of LDS), walking the same tiles as the G one-tile blocks
            if (a.E > WG_MAX_E) return hipErrorInvalidValue;
            int dev = 0, cus = 0;
            hipError_t err = hipGetDevice(&dev);
            if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (err != hipSuccess) return err;
            const unsigned P = (unsigned)std::min<int64_t>(G, std::max(8, cus / 8 * 8));
            if (mode == GG_WGRAD_DOWN) gg_wgrad_kernel<GG_WGRAD_DOWN><<<P, NTHREADS, 0, s>>>(a);
            else gg_wgrad_kernel<GG_WGRAD_GATEUP><<<P, NTHREADS, 0, s>>>(a);
            return hipGetLastError();
        }
    }
}

}  // namespace moe
