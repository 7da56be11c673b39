// Router: logits GEMM, softmax, wavefront top-K, capacity drop and permutation maps.
//
// "MoE Parallel Folding" (arXiv 2504.14960), knowledge-base notes page, method
// paragraph: the router assigns each token to its Top-K experts and a permutation
// makes one expert's tokens contiguous; Section 3.3 Token Dispatcher: assignments
// over capacity are dropped inside each sub-sequence.  Decisions are integer
// functions of fp32 values, so every floating-point step of the softmax is written
// out with its own rounding: no contraction (this file is built with
// -ffp-contract=off and the pragma below), IEEE division, pairwise sums.
#include "common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

// ---------------------------------------------------------------------------------
// exp for r <= 0: Cody & Waite range reduction (Software Manual for the Elementary
// Functions, 1980) with ln 2 = C1 + C2, C1 = ln 2 truncated to a multiple of 2^-16
// so n*C1 is exact, then the degree-7 Taylor polynomial in Horner form and an exact
// scaling by 2^n.  Results below 2^-125 are flushed to +0 (no denormal is made).
// ---------------------------------------------------------------------------------
constexpr double kLn2 = 0.69314718055994530942;
constexpr float kC1 = (float)(45426.0 / 65536.0);
constexpr float kC2 = (float)(kLn2 - 45426.0 / 65536.0);
constexpr float kInvLn2 = (float)(1.0 / kLn2);

__device__ __forceinline__ float route_exp(float r) {
    float t = r * kInvLn2;
    float n = __builtin_rintf(t);
    if (n < -125.0f) return 0.0f;
    float rr = r - n * kC1;
    rr = rr - n * kC2;
    float q = (float)(1.0 / 5040.0);
    q = q * rr + (float)(1.0 / 720.0);
    q = q * rr + (float)(1.0 / 120.0);
    q = q * rr + (float)(1.0 / 24.0);
    q = q * rr + (float)(1.0 / 6.0);
    q = q * rr + 0.5f;
    q = q * rr + 1.0f;
    q = q * rr + 1.0f;
    return q * __uint_as_float((uint32_t)((int)n + 127) << 23);
}

__device__ __forceinline__ int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Cross-lane exchange for the butterflies below, without the LDS crossbar.  Steps 1 and
// 2 are DPP quad permutations (lane i ^ m); steps 4 and 8 are DPP mirrors within rows of
// 16 (lane 7 - i within each 8, 15 - i within each 16): that partner lies in the other
// half of the same group of 2m lanes as i ^ m, so a reduction step combines the same
// two half-groups.  Steps 16 and 32 use the gfx950 lane swaps across rows and halves
// (v_permlane16_swap / v_permlane32_swap applied to two copies of v), which hand every
// lane its own value and its partner's i ^ m, in an order that depends on the lane; the
// reductions here are symmetric in the two, so both are passed on.
template <int M>
__device__ __forceinline__ uint32_t dpp_partner(uint32_t v) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8, "DPP steps");
    constexpr int ctrl = M == 1 ? 0xB1 : M == 2 ? 0x4E : M == 4 ? 0x141 : 0x140;
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xF, 0xF, false);
}
template <int M>
__device__ __forceinline__ void swap_pair(uint32_t v, uint32_t& a, uint32_t& b) {
    static_assert(M == 16 || M == 32, "lane-swap steps");
    if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        a = r[0], b = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        a = r[0], b = r[1];
    }
}

// One butterfly step of a sum: own value plus the partner's (fp addition is commutative,
// so the order of the two operands does not change the result).
template <int M>
__device__ __forceinline__ float sum_step(float v) {
    if constexpr (M <= 8) {
        return v + __uint_as_float(dpp_partner<M>(__float_as_uint(v)));
    } else {
        uint32_t a, b;
        swap_pair<M>(__float_as_uint(v), a, b);
        return __uint_as_float(a) + __uint_as_float(b);
    }
}

// Sum over lanes [0, P) by a butterfly (P a power of two, at most 64): every lane of the
// group ends with the pairwise-tree sum ((v0+v1)+(v2+v3))+..., the same value on every
// lane.
__device__ __forceinline__ float butterfly_sum(float v, int P) {
    if (P > 1) v = sum_step<1>(v);
    if (P > 2) v = sum_step<2>(v);
    if (P > 4) v = sum_step<4>(v);
    if (P > 8) v = sum_step<8>(v);
    if (P > 16) v = sum_step<16>(v);
    if (P > 32) v = sum_step<32>(v);
    return v;
}

template <int M>
__device__ __forceinline__ float max_step(float v) {
    if constexpr (M <= 8) {
        return fmaxf(v, __uint_as_float(dpp_partner<M>(__float_as_uint(v))));
    } else {
        uint32_t a, b;
        swap_pair<M>(__float_as_uint(v), a, b);
        return fmaxf(__uint_as_float(a), __uint_as_float(b));
    }
}

__device__ __forceinline__ float wave_max(float v) {
    v = max_step<1>(v);
    v = max_step<2>(v);
    v = max_step<4>(v);
    v = max_step<8>(v);
    v = max_step<16>(v);
    return max_step<32>(v);
}

// One step of the wave-wide maximum of the 64-bit key (hi, lo).
__device__ __forceinline__ void key_max(uint32_t& h, uint32_t& l, uint32_t oh, uint32_t ol) {
    const bool take = (oh > h) || (oh == h && ol > l);
    h = take ? oh : h;
    l = take ? ol : l;
}
template <int M>
__device__ __forceinline__ void key_step(uint32_t& h, uint32_t& l) {
    if constexpr (M <= 8) {
        key_max(h, l, dpp_partner<M>(h), dpp_partner<M>(l));
    } else {
        uint32_t h0, h1, l0, l1;
        swap_pair<M>(h, h0, h1);
        swap_pair<M>(l, l0, l1);
        h = h0, l = l0;
        key_max(h, l, h1, l1);
    }
}

// Softmax over E logits held one per lane (lane < E), top-K by (p desc, e asc),
// gates renormalised over the K chosen.  Writes the token's K slots.
__device__ void softmax_topk_token(float logit, int E, int K, int64_t t,
                                   int32_t* __restrict__ topk_idx, float* __restrict__ topk_prob,
                                   float* __restrict__ topk_gate) {
    const int lane = threadIdx.x & 63;
    const bool on = lane < E;
    float l = on ? logit : -INFINITY;
    float m = wave_max(l);
    float u = on ? route_exp(l - m) : 0.0f;
    float Z = butterfly_sum(u, next_pow2(E));
    float p = on ? u / Z : 0.0f;

    // K rounds of a wave-wide max over the 64-bit key (p bits, 0xFFFF - e).
    uint32_t khi = on ? __float_as_uint(p) : 0u;
    uint32_t klo = on ? (0xFFFFu - (uint32_t)lane) : 0u;
    int sel_e = 0;
    float sel_p = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint32_t bh = khi, bl = klo;
        key_step<1>(bh, bl);
        key_step<2>(bh, bl);
        key_step<4>(bh, bl);
        key_step<8>(bh, bl);
        key_step<16>(bh, bl);
        key_step<32>(bh, bl);
        int e = (int)(0xFFFFu - bl);
        if (lane == e) { khi = 0u; klo = 0u; }
        if (lane == k) { sel_e = e; sel_p = __uint_as_float(bh); }
    }
    float P = butterfly_sum(lane < K ? sel_p : 0.0f, next_pow2(K));
    if (lane < K) {
        topk_idx[t * K + lane] = sel_e;
        topk_prob[t * K + lane] = sel_p;
        topk_gate[t * K + lane] = sel_p / P;
    }
}

// ---------------------------------------------------------------------------------
// Router GEMM, bf16 on MFMA: a block of W waves takes 16 tokens; the waves split d
// (split-K, W = 8 when d % 256 == 0, else 4) and each computes 16 tokens x 16*NB expert
// columns with v_mfma_f32_16x16x32_bf16; the W partial sums are added in a fixed order
// in LDS. Column E (if present) is the shared expert's gate vector w_sg.  A wave's
// slice of d is short (768 k for d = 6144), so the kernel is bound by load latency
// unless many loads are in flight: a lane loads its x fragments and the matching
// weight fragments (L2-resident, shared by every block) of BL k-steps together, and the
// loads of the next BL k-steps are issued before the current ones are used (two
// register buffers).  Every wave adds its k-steps in ascending order, so the sums do not
// depend on BL.
// ---------------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int RT_TOK = 16;     // tokens per block
constexpr int RT_NBMAX = 5;    // up to 80 columns (64 experts + shared gate)

// w_frag: the router weight (and w_sg as column E, zero columns up to 16 NB) in the
// order the MFMA B fragments are read: for k-step s (32 k) and column block j, 1 KB of
// 64 lanes x 8 bf16, lane q holding column 16 j + (q & 15), k = 32 s + 8 (q >> 4) + 0..7.
// A wave's fragment load is then 1 KB of consecutive bytes (eight whole 128-byte lines)
// at a wave-uniform offset.
__global__ void __launch_bounds__(256) router_w_fragments(const bf16_t* __restrict__ w,
                                                          const bf16_t* __restrict__ w_sg,
                                                          bf16_t* __restrict__ w_frag, int d,
                                                          int E, int NB) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= (int64_t)NB * 16 * d) return;
    const int e8 = (int)(o & 7);
    const int q = (int)((o >> 3) & 63);
    const int64_t blk = o >> 9;
    const int j = (int)(blk % NB);
    const int64_t ks = blk / NB;
    const int col = 16 * j + (q & 15);
    const int64_t k = ks * 32 + 8 * (q >> 4) + e8;
    bf16_t v = 0;
    if (col < E) v = w[k * E + col];
    else if (col == E && w_sg) v = w_sg[k];
    w_frag[o] = v;
}

template <int W, int NB>
__global__ void __launch_bounds__(64 * W) router_fwd_mfma(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w_frag, const float* __restrict__ bias,
    float* __restrict__ logits, float* __restrict__ sg_logit, int T, int d, int E, int K,
    int has_sg, int32_t* __restrict__ topk_idx, float* __restrict__ topk_prob,
    float* __restrict__ topk_gate) {
    static_assert(NB >= 1 && NB <= RT_NBMAX, "1 to 5 column blocks");
    // k-steps per register buffer: (1 + NB) 16-byte loads per k-step and lane, two buffers
    constexpr int BL = NB <= 2 ? 8 : 4;
    __shared__ float part[W][RT_TOK][RT_NBMAX * 16 + 1];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int t0 = blockIdx.x * RT_TOK;
    const int row = lane & 15;      // token within the block (A) / column (B)
    const int kq = lane >> 4;       // which 8-wide k group of the 32
    const int dslice = d / W;       // a multiple of 32
    const int kbeg = wave * dslice;

    f32x4_t acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int tok = t0 + row;
    const bool tok_ok = tok < T;
    // Buffer loads: a per-lane byte offset and a wave-uniform one (the k-step, and for the
    // weight the column block) against a resource over the block's rows of x, or over the
    // transposed weight.  Rows past T read the block's first row and are zeroed.  A k-step
    // at or past the slice's end (loaded with its batch, never used) loads the slice's
    // last k-step again, so every access stays inside the wave's own slice.
    const int rows = min(RT_TOK, T - t0);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + (int64_t)t0 * d), 0, rows * d * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)w_frag, 0, NB * 16 * d * 2, 0x00020000);
    const int xo = ((tok_ok ? row : 0) * d + kbeg + kq * 8) * 2;
    const int wo = lane * 16;
    const int ks0 = kbeg / 32;  // the wave's first k-step

    // Loads of the BL k-steps from k.
    auto load = [&](u32x4 (&xv)[BL], u32x4 (&wv)[BL][NB], int k) {
#pragma unroll
        for (int u = 0; u < BL; ++u) {
            const int ku = min(k + 32 * u, dslice - 32);
            xv[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo, ku * 2, 0));
#pragma unroll
            for (int j = 0; j < NB; ++j)
                wv[u][j] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, wo, ((ks0 + ku / 32) * NB + j) * 1024, 0));
        }
    };
    auto compute = [&](const u32x4 (&xv)[BL], const u32x4 (&wv)[BL][NB], int k) {
#pragma unroll
        for (int u = 0; u < BL; ++u) {
            if (k + 32 * u < dslice) {
                const u32x4 az = tok_ok ? xv[u] : u32x4{0, 0, 0, 0};
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, az);
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a, __builtin_bit_cast(bf16x8_t, wv[u][j]), acc[j], 0, 0, 0);
            }
        }
    };
    // Two register buffers; the last batch is computed on its own branch, so that each
    // compute follows its loads' issue in straight-line code (the compiler then waits for
    // those loads only, not for the next batch's).
    u32x4 x0[BL], x1[BL], w0[BL][NB], w1[BL][NB];
    constexpr int KB = 32 * BL;
    load(x0, w0, 0);
    for (int k = 0;;) {
        if (k + KB >= dslice) { compute(x0, w0, k); break; }
        load(x1, w1, k + KB);
        compute(x0, w0, k);
        k += KB;
        if (k + KB >= dslice) { compute(x1, w1, k); break; }
        load(x0, w0, k + KB);
        compute(x1, w1, k);
        k += KB;
    }
    // D layout of the 16x16 MFMA: lane holds column (lane & 15), rows 4*(lane>>4)+i.
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][4 * kq + i][j * 16 + row] = acc[j][i];
    __syncthreads();
    // Each wave finishes RT_TOK / W tokens: fixed-order sum of the W split-K partials,
    // bias, then softmax and top-K with one lane per expert.
    auto colsum = [&](int tl, int c) {
        float v = part[0][tl][c];
#pragma unroll
        for (int w = 1; w < W; ++w) v += part[w][tl][c];
        return v;
    };
    for (int q = 0; q < RT_TOK / W; ++q) {
        int tl = wave * (RT_TOK / W) + q;
        int t = t0 + tl;
        if (t >= T) break;
        float l = 0.f;
        if (lane < E) {
            l = colsum(tl, lane);
            if (bias) l = l + bias[lane];
            logits[(int64_t)t * E + lane] = l;
        }
        // the shared gate is column E, which can be past the last lane (E = 64)
        if (has_sg && lane == 0) sg_logit[t] = colsum(tl, E);
        softmax_topk_token(l, E, K, t, topk_idx, topk_prob, topk_gate);
    }
}

// Generic router (fp32, or bf16 with d % 128 != 0): one wave per token.
template <typename T>
__global__ void __launch_bounds__(64) router_fwd_valu(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ bias,
    const T* __restrict__ w_sg, float* __restrict__ logits, float* __restrict__ sg_logit,
    int d, int E, int K, int32_t* __restrict__ topk_idx, float* __restrict__ topk_prob,
    float* __restrict__ topk_gate) {
    __shared__ float lg[65];
    const int lane = threadIdx.x;
    const int64_t t = blockIdx.x;
    const int ncol = E + (w_sg ? 1 : 0);
    for (int e = 0; e < ncol; ++e) {
        float s = 0.f;
        for (int k = lane; k < d; k += 64) {
            float wv = (e < E) ? Elem<T>::load(w, (int64_t)k * E + e) : Elem<T>::load(w_sg, k);
            s += Elem<T>::load(x, t * d + k) * wv;
        }
        s = wave_sum(s);
        if (lane == 0) lg[e] = s;
    }
    __syncthreads();
    float l = 0.f;
    if (lane < E) {
        l = lg[lane];
        if (bias) l = l + bias[lane];
        logits[t * E + lane] = l;
    }
    if (w_sg && lane == 0) sg_logit[t] = lg[E];  // column E can be past the last lane
    softmax_topk_token(l, E, K, t, topk_idx, topk_prob, topk_gate);
}

__global__ void __launch_bounds__(256) topk_from_logits(const float* __restrict__ logits, int T,
                                                        int E, int K,
                                                        int32_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_prob,
                                                        float* __restrict__ topk_gate) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    float l = lane < E ? logits[t * E + lane] : 0.f;
    softmax_topk_token(l, E, K, t, topk_idx, topk_prob, topk_gate);
}

// ---------------------------------------------------------------------------------
// Capacity drop, one block per (sub-sequence s, expert e).  The candidates are the
// tokens of the sub-sequence that chose e (at most one slot each), collected in
// token order.  If there are more than `capacity`, the kept ones are the capacity
// largest under (p desc, t asc): a 4-pass radix select on the fp32 bit pattern of
// p (order-preserving for p >= 0) finds the threshold value and how many of the
// candidates equal to it are kept; those are the first ones in token order.
// ---------------------------------------------------------------------------------
constexpr int SEL_THREADS = 1024;  // one block per (sub-sequence, expert): few blocks, wide

__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int* total) {
    // sh: >= SEL_THREADS / 64 ints of shared memory
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(incl, o, MOE_WAVE);
        if (lane >= o) incl += n;
    }
    __syncthreads();
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < SEL_THREADS / 64; ++w) {
        if (w < wave) base += sh[w];
        tot += sh[w];
    }
    *total = tot;
    return base + incl - v;
}

__global__ void __launch_bounds__(SEL_THREADS) select_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_prob, int S, int E,
    int K, int capacity, uint8_t* __restrict__ keep, int32_t* __restrict__ row_of,
    int32_t* __restrict__ routed_counts, int32_t* __restrict__ kcnt, int32_t* __restrict__ cand,
    int32_t* __restrict__ kept_list) {
    __shared__ int sh_scan[SEL_THREADS / 64];
    __shared__ int hist[256];
    __shared__ int sh_digit, sh_above;
    const int s = blockIdx.y;
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    const int per = (S + SEL_THREADS - 1) / SEL_THREADS;
    const int64_t tbeg = (int64_t)s * S + (int64_t)tid * per;
    const int64_t tend = min(tbeg + per, (int64_t)(s + 1) * S);
    const int64_t g = (int64_t)s * E + e;
    int32_t* my_cand = cand + g * S;
    int32_t* my_kept = kept_list + g * S;

    int c = 0;
    for (int64_t t = tbeg; t < tend; ++t)
        for (int k = 0; k < K; ++k)
            if (topk_idx[t * K + k] == e) ++c;
    int n;
    int base = block_exclusive_scan(c, sh_scan, &n);
    {
        int w = base;
        for (int64_t t = tbeg; t < tend; ++t)
            for (int k = 0; k < K; ++k)
                if (topk_idx[t * K + k] == e) my_cand[w++] = (int32_t)(t * K + k);
    }
    if (tid == 0) routed_counts[g] = n;

    // Threshold (bits of the capacity-th largest p) and how many equal to it to keep.
    uint32_t thr = 0u;
    int want_eq = 0;
    const bool all_kept = capacity < 0 || n <= capacity;
    const bool none_kept = !all_kept && capacity == 0;
    if (!all_kept && !none_kept) {
        uint32_t prefix = 0u, pmask = 0u;
        int want = capacity;
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
            __syncthreads();
            for (int i = base; i < base + c; ++i) {
                uint32_t key = __float_as_uint(topk_prob[my_cand[i]]);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
            }
            __syncthreads();
            if (tid < 64) {
                // lane l owns digits 255-4l .. 252-4l (descending)
                int hv[4];
                int loc = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) { hv[j] = hist[255 - 4 * tid - j]; loc += hv[j]; }
                int incl = loc;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    int nb = __shfl_up(incl, o, MOE_WAVE);
                    if (tid >= o) incl += nb;
                }
                int excl = incl - loc;  // count of digits above this lane's four
                bool hit = excl < want && incl >= want;
                if (hit) {
                    int run = excl;
                    for (int j = 0; j < 4; ++j) {
                        if (run + hv[j] >= want) {
                            sh_digit = 255 - 4 * tid - j;
                            sh_above = run;
                            break;
                        }
                        run += hv[j];
                    }
                }
            }
            __syncthreads();
            want -= sh_above;
            prefix |= ((uint32_t)sh_digit) << shift;
            pmask |= 255u << shift;
            __syncthreads();
        }
        thr = prefix;
        want_eq = want;
    }

    // Keep flags, in token order; equal-to-threshold candidates ranked by token.
    int eq_local = 0;
    if (!all_kept && !none_kept)
        for (int i = base; i < base + c; ++i)
            if (__float_as_uint(topk_prob[my_cand[i]]) == thr) ++eq_local;
    int eq_tot;
    int eq_base = block_exclusive_scan(eq_local, sh_scan, &eq_tot);
    int kc = 0;
    {
        int eq_seen = eq_base;
        for (int i = base; i < base + c; ++i) {
            int slot = my_cand[i];
            bool kp;
            if (all_kept) kp = true;
            else if (none_kept) kp = false;
            else {
                uint32_t key = __float_as_uint(topk_prob[slot]);
                if (key > thr) kp = true;
                else if (key == thr) kp = (eq_seen++ < want_eq);
                else kp = false;
            }
            keep[slot] = kp ? 1 : 0;
            if (!kp) row_of[slot] = -1;
            kc += kp ? 1 : 0;
        }
    }
    int ktot;
    int kbase = block_exclusive_scan(kc, sh_scan, &ktot);
    {
        int w = kbase;
        for (int i = base; i < base + c; ++i) {
            int slot = my_cand[i];
            if (keep[slot]) my_kept[w++] = slot;
        }
    }
    if (tid == 0) kcnt[g] = ktot;
}

// The same selection with each thread's candidates held in registers (a sub-sequence
// of at most SEL_THREADS * PER tokens, PER = 16 or 32): thread i owns tokens
// i*per .. i*per+per-1 and has at most one candidate slot per token, so candidate j of
// the thread sits at the fixed register index j and every pass reads registers instead
// of global memory.
constexpr int SEL_PER = 16;

template <int PER>
__global__ void __launch_bounds__(SEL_THREADS) select_kernel_reg(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_prob, int S, int E,
    int K, int capacity, uint8_t* __restrict__ keep, int32_t* __restrict__ row_of,
    int32_t* __restrict__ routed_counts, int32_t* __restrict__ kcnt,
    int32_t* __restrict__ kept_list) {
    __shared__ int sh_scan[SEL_THREADS / 64];
    __shared__ int hist[256];
    __shared__ int sh_digit, sh_above;
    const int s = blockIdx.y;
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    const int per = (S + SEL_THREADS - 1) / SEL_THREADS;
    const int64_t tbeg = (int64_t)s * S + (int64_t)tid * per;
    const int64_t tend = min(tbeg + per, (int64_t)(s + 1) * S);
    const int64_t g = (int64_t)s * E + e;
    int32_t* my_kept = kept_list + g * S;

    int slot[PER];
    uint32_t key[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        slot[j] = -1;
        const int64_t t = tbeg + j;
        if (j < per && t < tend)
            for (int k = 0; k < K; ++k)
                if (topk_idx[t * K + k] == e) slot[j] = (int)(t * K + k);
    }
    int c = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        key[j] = slot[j] >= 0 ? __float_as_uint(topk_prob[slot[j]]) : 0u;
        c += slot[j] >= 0 ? 1 : 0;
    }
    int n;
    block_exclusive_scan(c, sh_scan, &n);
    if (tid == 0) routed_counts[g] = n;

    uint32_t thr = 0u;
    int want_eq = 0;
    const bool all_kept = capacity < 0 || n <= capacity;
    const bool none_kept = !all_kept && capacity == 0;
    if (!all_kept && !none_kept) {
        uint32_t prefix = 0u, pmask = 0u;
        int want = capacity;
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if (slot[j] >= 0 && (key[j] & pmask) == prefix)
                    atomicAdd(&hist[(key[j] >> shift) & 255u], 1);
            __syncthreads();
            if (tid < 64) {
                // lane l owns digits 255-4l .. 252-4l (descending)
                int hv[4];
                int loc = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) { hv[q] = hist[255 - 4 * tid - q]; loc += hv[q]; }
                int incl = loc;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    int nb = __shfl_up(incl, o, MOE_WAVE);
                    if (tid >= o) incl += nb;
                }
                int excl = incl - loc;
                if (excl < want && incl >= want) {
                    int run = excl;
                    for (int q = 0; q < 4; ++q) {
                        if (run + hv[q] >= want) {
                            sh_digit = 255 - 4 * tid - q;
                            sh_above = run;
                            break;
                        }
                        run += hv[q];
                    }
                }
            }
            __syncthreads();
            want -= sh_above;
            prefix |= ((uint32_t)sh_digit) << shift;
            pmask |= 255u << shift;
            __syncthreads();
        }
        thr = prefix;
        want_eq = want;
    }

    // keep flags in token order; candidates equal to the threshold ranked by token
    int eq_local = 0;
    if (!all_kept && !none_kept) {
#pragma unroll
        for (int j = 0; j < PER; ++j) eq_local += (slot[j] >= 0 && key[j] == thr) ? 1 : 0;
    }
    int eq_tot;
    int eq_seen = block_exclusive_scan(eq_local, sh_scan, &eq_tot);
    uint32_t kept_mask = 0u;
    int kc = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (slot[j] < 0) continue;
        bool kp;
        if (all_kept) kp = true;
        else if (none_kept) kp = false;
        else if (key[j] > thr) kp = true;
        else if (key[j] == thr) kp = (eq_seen++ < want_eq);
        else kp = false;
        keep[slot[j]] = kp ? 1 : 0;
        if (!kp) row_of[slot[j]] = -1;
        kept_mask |= kp ? (1u << j) : 0u;
        kc += kp ? 1 : 0;
    }
    int ktot;
    int w = block_exclusive_scan(kc, sh_scan, &ktot);
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (kept_mask & (1u << j)) my_kept[w++] = slot[j];
    if (tid == 0) kcnt[g] = ktot;
}

// Rows of every kept assignment: experts in ascending order, then tokens ascending
// (sub-sequences in order, token order inside each).  One block per (s, e).
__global__ void __launch_bounds__(256) maps_kernel(const int32_t* __restrict__ kcnt,
                                                   const int32_t* __restrict__ kept_list,
                                                   int n_sub, int S, int E,
                                                   int32_t* __restrict__ row_of,
                                                   int32_t* __restrict__ src_of,
                                                   int32_t* __restrict__ kept_counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ n_kept) {
    __shared__ int red[4];
    const int s = blockIdx.y;
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    // base = kept rows of experts < e (all sub-sequences) + of expert e in sub-seqs < s
    int part = 0;
    for (int i = tid; i < n_sub * E; i += 256) {
        int ss = i / E, ee = i % E;
        if (ee < e || (ee == e && ss < s)) part += kcnt[i];
    }
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, MOE_WAVE);
    if ((tid & 63) == 0) red[tid >> 6] = part;
    __syncthreads();
    const int base = red[0] + red[1] + red[2] + red[3];
    const int64_t g = (int64_t)s * E + e;
    const int cnt = kcnt[g];
    const int32_t* lst = kept_list + g * S;
    for (int j = tid; j < cnt; j += 256) {
        int slot = lst[j];
        src_of[base + j] = slot;
        row_of[slot] = base + j;
    }
    if (s == 0 && e == 0 && tid < 64) {
        // kept counts per expert and their exclusive scan (E <= 64: one lane each)
        int kc = 0;
        if (tid < E)
            for (int ss = 0; ss < n_sub; ++ss) kc += kcnt[(int64_t)ss * E + tid];
        int incl = kc;
        for (int o = 1; o < 64; o <<= 1) {
            int nb = __shfl_up(incl, o, MOE_WAVE);
            if (tid >= o) incl += nb;
        }
        if (tid < E) {
            kept_counts[tid] = kc;
            offsets[tid] = incl - kc;
        }
        if (tid == E - 1) {
            offsets[E] = incl;
            n_kept[0] = incl;
        }
    }
}

}  // namespace

hipError_t launch_router_fwd(const moe_desc& d, const void* x, const void* w_router,
                             const float* bias, const void* w_sg, float* logits,
                             float* sg_logit, const moe_routing& r, hipStream_t s,
                             void* w_rt_ws) {
    const int ncol = d.E + (w_sg ? 1 : 0);
    if (d.dtype == MOE_BF16 && d.d % 128 == 0 && w_rt_ws) {
        const int NB = (ncol + 15) / 16;
        bf16_t* wrt = (bf16_t*)w_rt_ws;
        int64_t n = (int64_t)NB * 16 * d.d;
        router_w_fragments<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            (const bf16_t*)w_router, (const bf16_t*)w_sg, wrt, d.d, d.E, NB);
        const unsigned nb = (d.T + RT_TOK - 1) / RT_TOK;
        auto launch = [&](auto w_tag, auto nb_tag) {
            constexpr int W = decltype(w_tag)::value, NBc = decltype(nb_tag)::value;
            router_fwd_mfma<W, NBc><<<nb, 64 * W, 0, s>>>(
                (const bf16_t*)x, wrt, bias, logits, sg_logit, d.T, d.d, d.E, d.K,
                w_sg ? 1 : 0, r.topk_idx, r.topk_prob, r.topk_gate);
        };
        auto by_nb = [&](auto w_tag) {
            switch (NB) {
                case 1: launch(w_tag, std::integral_constant<int, 1>{}); break;
                case 2: launch(w_tag, std::integral_constant<int, 2>{}); break;
                case 3: launch(w_tag, std::integral_constant<int, 3>{}); break;
                case 4: launch(w_tag, std::integral_constant<int, 4>{}); break;
                default: launch(w_tag, std::integral_constant<int, 5>{}); break;
            }
        };
        if (d.d % 256 == 0) by_nb(std::integral_constant<int, 8>{});
        else by_nb(std::integral_constant<int, 4>{});
    } else if (d.dtype == MOE_BF16) {
        router_fwd_valu<bf16_t><<<d.T, 64, 0, s>>>(
            (const bf16_t*)x, (const bf16_t*)w_router, bias, (const bf16_t*)w_sg, logits, sg_logit,
            d.d, d.E, d.K, r.topk_idx, r.topk_prob, r.topk_gate);
    } else {
        router_fwd_valu<float><<<d.T, 64, 0, s>>>(
            (const float*)x, (const float*)w_router, bias, (const float*)w_sg, logits, sg_logit,
            d.d, d.E, d.K, r.topk_idx, r.topk_prob, r.topk_gate);
    }
    return hipGetLastError();
}

hipError_t launch_topk_from_logits(const moe_desc& d, const float* logits, const moe_routing& r,
                                   hipStream_t s) {
    topk_from_logits<<<(d.T + 3) / 4, 256, 0, s>>>(logits, d.T, d.E, d.K, r.topk_idx,
                                                   r.topk_prob, r.topk_gate);
    return hipGetLastError();
}

hipError_t launch_select_and_maps(const moe_desc& d, const moe_routing& r, RouteWs ws,
                                  hipStream_t s) {
    const int n_sub = d.T / d.sub_seq;
    dim3 grid(d.E, n_sub);
    int32_t* cand = ws.list;
    int32_t* kept = ws.list + (int64_t)n_sub * d.E * d.sub_seq;
    if (d.sub_seq <= SEL_THREADS * SEL_PER)
        select_kernel_reg<SEL_PER><<<grid, SEL_THREADS, 0, s>>>(
            r.topk_idx, r.topk_prob, d.sub_seq, d.E, d.K, d.capacity, r.keep, r.row_of,
            r.routed_counts, ws.kcnt, kept);
    else if (d.sub_seq <= SEL_THREADS * 2 * SEL_PER)
        select_kernel_reg<2 * SEL_PER><<<grid, SEL_THREADS, 0, s>>>(
            r.topk_idx, r.topk_prob, d.sub_seq, d.E, d.K, d.capacity, r.keep, r.row_of,
            r.routed_counts, ws.kcnt, kept);
    else
        select_kernel<<<grid, SEL_THREADS, 0, s>>>(r.topk_idx, r.topk_prob, d.sub_seq, d.E, d.K,
                                                   d.capacity, r.keep, r.row_of, r.routed_counts,
                                                   ws.kcnt, cand, kept);
    maps_kernel<<<grid, 256, 0, s>>>(ws.kcnt, kept, n_sub, d.sub_seq, d.E, r.row_of, r.src_of,
                                     r.kept_counts, r.offsets, r.n_kept);
    return hipGetLastError();
}

}  // namespace moe
