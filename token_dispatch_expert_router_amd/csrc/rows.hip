// Row movement of the dispatcher and its backward duals, plus the router backward.
//
// "MoE Parallel Folding" (arXiv 2504.14960), knowledge-base notes page, method
// paragraph: permutation gathers each expert's tokens into a contiguous block, the
// un-permutation restores token order, and the backward pass runs the duals.  These
// kernels are pure HBM streams: every row is moved with 16-byte vector accesses, one
// wavefront per token (the permute backward with few experts: one column slice of many
// tokens per block), with a batch of loads in flight per lane.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

constexpr int ROWS_PER_BLOCK = 4;  // one wave per row, 4 waves per block

// Chunks of a row handled by one lane per batch: lane handles chunks c0 + lane + 64u,
// u < CHUNKS, and issues the loads of a whole batch before using any of them, so that
// every lane keeps CHUNKS 16-byte loads in flight per source row (rows of d = 6144 bf16
// are three batches).  4 measured best (permute 6% faster than 6; 8 and 12 slower, and
// nontemporal accesses 10-25% slower).
constexpr int CHUNKS = 4;

// A batch that lies wholly inside the row (FULL) is loaded and stored without per-chunk
// predicates, so that all its loads issue back to back; in the row's last partial batch a
// chunk past the row reads the row's last chunk instead (a valid address; its value is
// never stored), so the loads stay unconditional there too and the batch stays in
// registers.
template <bool FULL, int U>
__device__ __forceinline__ void load_batch(const u32x4* __restrict__ row, int c0, int lane, int vpr,
                                           u32x4 (&v)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + 64 * u;
        v[u] = row[FULL ? c : min(c, vpr - 1)];
    }
}

// Runs body(c0, std::integral_constant<bool, FULL>) for every batch of U chunks per lane.
template <int U = CHUNKS, typename F>
__device__ __forceinline__ void for_batches(int vpr, F&& body) {
    int c0 = 0;
    for (; c0 + 64 * U <= vpr; c0 += 64 * U) body(c0, std::true_type{});
    if (c0 < vpr) body(c0, std::false_type{});
}

// The token a wave works on, as a wave-uniform value: its per-slot routing entries are
// then read with scalar loads inside the loops instead of being kept in arrays.
__device__ __forceinline__ int64_t wave_token() {
    return __builtin_amdgcn_readfirstlane((int)(blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6)));
}

// acc[u] += w * row[c0 + lane + 64u] for one batch.
template <typename T, bool FULL>
__device__ __forceinline__ void add_batch(const u32x4* __restrict__ row, float w, int c0, int lane,
                                          int vpr, float (&acc)[CHUNKS][Vec16<T>::N]) {
    constexpr int N = Vec16<T>::N;
    u32x4 v[CHUNKS];
    load_batch<FULL>(row, c0, lane, vpr, v);
#pragma unroll
    for (int u = 0; u < CHUNKS; ++u) {
        float f[N];
        Vec16<T>::unpack(v[u], f);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[u][i] += w * f[i];
    }
}

// The routing entries of a wave's token sit one slot per lane (lane k < K holds slot k),
// read with one vector load per array as the wave starts; a slot's row (-1 when the slot
// was dropped) and gate are then taken out with readlane as wave-uniform values, so that
// the row loads of every slot of a batch can be issued together instead of each waiting
// for its own routing entry.
__device__ __forceinline__ int lane_slot_row(const int32_t* __restrict__ row_of, int64_t t, int K,
                                             int lane) {
    return lane < K ? row_of[t * K + lane] : -1;
}
__device__ __forceinline__ float lane_slot_gate(const float* __restrict__ gate, int64_t t, int K,
                                                int lane) {
    return lane < K ? gate[t * K + lane] : 0.f;
}
__device__ __forceinline__ int slot_of(int v, int k) { return __builtin_amdgcn_readlane(v, k); }
__device__ __forceinline__ float slot_of(float v, int k) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
}

// Chunks per lane per batch of the one-token-per-wave kernels, by the most slots a token
// has (KM): every batch keeps KM * C (+ dy or shared) 16-byte loads per lane in flight.
template <int KM> struct RowBatch { static constexpr int C = KM <= 2 ? 6 : KM <= 4 ? 3 : 2; };

// xp[row_of[t,k]] = x[t] for every kept slot (t, k): token-major, so that each row of x
// is read once and stored to its kept rows (the same xp as gathering xp[r] =
// x[src_of[r] / K] row by row, with half the reads at K = 2).  The loads of x do not wait
// for the routing entries.
template <int KM>
__global__ void __launch_bounds__(256) permute_kernel(const u32x4* __restrict__ x,
                                                      const int32_t* __restrict__ row_of, int ntok,
                                                      int K, int vpr, u32x4* __restrict__ xp) {
    constexpr int C = RowBatch<2>::C;
    const int lane = threadIdx.x & 63;
    const int64_t t = wave_token();
    if (t >= ntok) return;
    const int rv = lane_slot_row(row_of, t, K, lane);
    const u32x4* src = x + t * vpr;
    for_batches<C>(vpr, [&](int c0, auto full) {
        constexpr bool FULL = decltype(full)::value;
        u32x4 v[C];
        load_batch<FULL>(src, c0, lane, vpr, v);
        // Keep the batch's loads here, once: every store of them sits under a per-slot
        // branch, into which the compiler would otherwise sink (and so repeat) the loads,
        // behind the wait for the routing entries.  The empty asm takes the values as
        // inputs, so the loads are issued before it and the routing load overlaps them.
#pragma unroll
        for (int u = 0; u < C; ++u) asm volatile("" ::"v"(v[u].x), "v"(v[u].y), "v"(v[u].z), "v"(v[u].w));
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            if (k >= K) break;
            const int row = slot_of(rv, k);
            if (row < 0) continue;
            u32x4* dst = xp + (int64_t)row * vpr;
#pragma unroll
            for (int u = 0; u < C; ++u) {
                const int c = c0 + lane + 64 * u;
                if (FULL || c < vpr) dst[c] = v[u];
            }
        }
    });
}

// y_t = sum_{kept k, ascending} g_tk o[row_of[t,k]]  (+ sigmoid(z_t) shared_t), fp32.
// Each batch issues the loads of every kept slot (and of the shared row) before adding any.
template <typename T, int KM>
__global__ void __launch_bounds__(256) unpermute_kernel(
    const u32x4* __restrict__ o, const int32_t* __restrict__ row_of,
    const float* __restrict__ gate, const u32x4* __restrict__ shared, const float* __restrict__ z,
    int ntok, int K, int vpr, u32x4* __restrict__ y) {
    constexpr int N = Vec16<T>::N;
    constexpr int C = RowBatch<KM>::C;
    const int lane = threadIdx.x & 63;
    const int64_t t = wave_token();
    if (t >= ntok) return;
    const int rv = lane_slot_row(row_of, t, K, lane);
    const float gv = lane_slot_gate(gate, t, K, lane);
    const float s = shared ? sigmoid_f(z[t]) : 0.f;
    for_batches<C>(vpr, [&](int c0, auto full) {
        constexpr bool FULL = decltype(full)::value;
        u32x4 v[KM][C], vs[C];
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            if (k >= K) break;
            const int row = slot_of(rv, k);
            if (row >= 0) load_batch<FULL>(o + (int64_t)row * vpr, c0, lane, vpr, v[k]);
        }
        if (shared) load_batch<FULL>(shared + t * vpr, c0, lane, vpr, vs);
        float acc[C][N];
#pragma unroll
        for (int u = 0; u < C; ++u)
#pragma unroll
            for (int i = 0; i < N; ++i) acc[u][i] = 0.f;
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            if (k >= K) break;
            if (slot_of(rv, k) < 0) continue;
            const float w = slot_of(gv, k);
#pragma unroll
            for (int u = 0; u < C; ++u) {
                float f[N];
                Vec16<T>::unpack(v[k][u], f);
#pragma unroll
                for (int i = 0; i < N; ++i) acc[u][i] += w * f[i];
            }
        }
        if (shared) {
#pragma unroll
            for (int u = 0; u < C; ++u) {
                float f[N];
                Vec16<T>::unpack(vs[u], f);
#pragma unroll
                for (int i = 0; i < N; ++i) acc[u][i] += s * f[i];
            }
        }
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const int c = c0 + lane + 64 * u;
            if (FULL || c < vpr) y[t * vpr + c] = Vec16<T>::pack(acc[u]);
        }
    });
}

// d_o[row_of[t,k]] = g_tk dy_t ; dgate_tk = <dy_t, o[row_of[t,k]]> ;
// shared: dshared_t = s_t dy_t, dz_t = <dy_t, shared_t> s_t (1 - s_t).
// Each batch loads dy and every kept slot's o piece (and the shared piece) together; the
// per-slot dot products stay in registers (KM of them).
template <typename T, int KM>
__global__ void __launch_bounds__(256) unpermute_bwd_kernel(
    const u32x4* __restrict__ dy, const u32x4* __restrict__ o, const int32_t* __restrict__ row_of,
    const float* __restrict__ gate, const u32x4* __restrict__ shared, const float* __restrict__ z,
    int ntok, int K, int vpr, u32x4* __restrict__ d_o, float* __restrict__ dgate,
    u32x4* __restrict__ dshared, float* __restrict__ dz) {
    constexpr int N = Vec16<T>::N;
    constexpr int C = RowBatch<KM>::C;
    const int lane = threadIdx.x & 63;
    const int64_t t = wave_token();
    if (t >= ntok) return;
    const int rv = lane_slot_row(row_of, t, K, lane);
    const float gv = lane_slot_gate(gate, t, K, lane);
    const float s = shared ? sigmoid_f(z[t]) : 0.f;
    float dot[KM], sdot = 0.f;
#pragma unroll
    for (int k = 0; k < KM; ++k) dot[k] = 0.f;
    // dot += <dy, r> over one batch; out = w * dy
    auto pair = [&](auto full, const u32x4 (&dvr)[C], const u32x4 (&rv_)[C], float w,
                    u32x4* __restrict__ out, int c0) -> float {
        constexpr bool FULL = decltype(full)::value;
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const int c = c0 + lane + 64 * u;
            if (!FULL && c >= vpr) continue;
            float dv[N], rf[N], wv[N];
            Vec16<T>::unpack(dvr[u], dv);
            Vec16<T>::unpack(rv_[u], rf);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                acc += dv[i] * rf[i];
                wv[i] = w * dv[i];
            }
            out[c] = Vec16<T>::pack(wv);
        }
        return acc;
    };
    for_batches<C>(vpr, [&](int c0, auto full) {
        constexpr bool FULL = decltype(full)::value;
        u32x4 dvr[C], v[KM][C], vs[C];
        load_batch<FULL>(dy + t * vpr, c0, lane, vpr, dvr);
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            if (k >= K) break;
            const int row = slot_of(rv, k);
            if (row >= 0) load_batch<FULL>(o + (int64_t)row * vpr, c0, lane, vpr, v[k]);
        }
        if (shared) load_batch<FULL>(shared + t * vpr, c0, lane, vpr, vs);
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            if (k >= K) break;
            const int row = slot_of(rv, k);
            if (row < 0) continue;
            dot[k] += pair(full, dvr, v[k], slot_of(gv, k), d_o + (int64_t)row * vpr, c0);
        }
        if (shared) sdot += pair(full, dvr, vs, s, dshared + t * vpr, c0);
    });
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        if (k >= K) break;
        const float v = slot_of(rv, k) >= 0 ? wave_sum(dot[k]) : 0.f;
        if (lane == 0) dgate[t * K + k] = v;
    }
    if (shared) {
        // sigma'(z) = sigma(z) sigma(-z): 1 - s would lose the leading bits of sigma(-z)
        // when s is close to 1
        const float v = wave_sum(sdot);
        if (lane == 0) dz[t] = v * s * sigmoid_f(-z[t]);
    }
}

// w_rt[e][i] = w_router[i][e] (e < E), w_rt[E][i] = w_sg[i]: row access for the
// router term of dx.
template <typename T>
__global__ void __launch_bounds__(256) transpose_rw_kernel(const T* __restrict__ w,
                                                           const T* __restrict__ w_sg,
                                                           T* __restrict__ w_rt, int d, int E,
                                                           int ncol) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)ncol * d) return;
    int e = (int)(i / d), k = (int)(i % d);
    T v = 0;
    if (e < E) {
        if (w) v = w[(int64_t)k * E + e];
    } else if (w_sg) {
        v = w_sg[k];
    }
    w_rt[i] = v;
}

// dx_t = sum_{kept k} dxp[row_of[t,k]] + sum_k dl[t,e_k] w_rt[e_k] + dz_t w_sg + dx_add_t
// (terms added in this order), one wave per token over its whole row, the router term from
// the transposed weight rows (L2-resident).  Used for many experts, where a block's slice
// of the router weight would take too much LDS for the slice kernel below.  The token's
// slots and its dlogits row sit one per lane; each batch issues the loads of every kept
// dxp piece (and dx_add) together, then those of the K router-weight rows.
template <typename T, int KM>
__global__ void __launch_bounds__(256) permute_bwd_rows_kernel(
    const u32x4* __restrict__ dxp, const int32_t* __restrict__ row_of,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ dlogits,
    const u32x4* __restrict__ w_rt, const float* __restrict__ dz, const u32x4* __restrict__ dx_add,
    int ntok, int E, int K, int vpr, u32x4* __restrict__ dx) {
    constexpr int N = Vec16<T>::N;
    constexpr int C = RowBatch<KM>::C;
    const int lane = threadIdx.x & 63;
    const int64_t t = wave_token();
    if (t >= ntok) return;
    const int rv = lane_slot_row(row_of, t, K, lane);
    const int ev = lane < K ? topk_idx[t * K + lane] : 0;
    const float dl = dlogits && lane < E ? dlogits[t * E + lane] : 0.f;  // lane e: dl[t, e]
    const float zt = dz ? dz[t] : 0.f;
    for_batches<C>(vpr, [&](int c0, auto full) {
        constexpr bool FULL = decltype(full)::value;
        u32x4 v[KM][C], va[C];
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            if (k >= K) break;
            const int row = slot_of(rv, k);
            if (row >= 0) load_batch<FULL>(dxp + (int64_t)row * vpr, c0, lane, vpr, v[k]);
        }
        if (dx_add) load_batch<FULL>(dx_add + t * vpr, c0, lane, vpr, va);
        float acc[C][N];
#pragma unroll
        for (int u = 0; u < C; ++u)
#pragma unroll
            for (int i = 0; i < N; ++i) acc[u][i] = 0.f;
        auto add = [&](const u32x4 (&src)[C], float w) {
#pragma unroll
            for (int u = 0; u < C; ++u) {
                float f[N];
                Vec16<T>::unpack(src[u], f);
#pragma unroll
                for (int i = 0; i < N; ++i) acc[u][i] += w * f[i];
            }
        };
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            if (k >= K) break;
            if (slot_of(rv, k) >= 0) add(v[k], 1.0f);
        }
        if (dlogits) {
#pragma unroll
            for (int k = 0; k < KM; ++k) {
                if (k >= K) break;
                load_batch<FULL>(w_rt + (int64_t)slot_of(ev, k) * vpr, c0, lane, vpr, v[k]);
            }
#pragma unroll
            for (int k = 0; k < KM; ++k) {
                if (k >= K) break;
                add(v[k], slot_of(dl, slot_of(ev, k)));
            }
        }
        if (dz) {
            load_batch<FULL>(w_rt + (int64_t)E * vpr, c0, lane, vpr, v[0]);
            add(v[0], zt);
        }
        if (dx_add) add(va, 1.0f);
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const int c = c0 + lane + 64 * u;
            if (FULL || c < vpr) dx[t * vpr + c] = Vec16<T>::pack(acc[u]);
        }
    });
}

// dx_t = sum_{kept k} dxp[row_of[t,k]] + sum_k dl[t,e_k] w_router[:,e_k] + dz_t w_sg + dx_add_t
// (terms added in this order).
//
// A block owns one column slice (64 chunks of 16 bytes: lane i holds chunk i of the slice)
// and a run of tokens.  The slice of the router weight, transposed to [column e][i], and
// of w_sg sit in LDS, loaded once per block from w_router's own [d, E] layout, so that the
// router term of every token is an LDS read instead of a row fetched from L2.  A wave
// reads the routing entries of a window of 64 / KM tokens with one vector load per array
// (lane j holds slot j % KM of token j / KM) and takes them out with readlane, then walks
// the window U tokens at a time, issuing the loads of all U tokens' kept dxp pieces (and
// dx_add pieces) before using any of them.
//   KM: the largest K the instantiation handles (U * KM = 8 row pieces in flight);
//   NC: the LDS columns it holds (E, plus w_sg).
template <typename T, int KM, int NC>
__global__ void __launch_bounds__(256) permute_bwd_kernel(
    const u32x4* __restrict__ dxp, const int32_t* __restrict__ row_of,
    const uint8_t* __restrict__ keep, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ dlogits, const T* __restrict__ w_router,
    const float* __restrict__ dz, const T* __restrict__ w_sg, const u32x4* __restrict__ dx_add,
    int ntok, int d, int E, int K, int vpr, int n_slices, int tok_per_block,
    u32x4* __restrict__ dx) {
    constexpr int N = Vec16<T>::N;   // elements per chunk
    constexpr int SW = 64 * N;       // columns of a slice
    constexpr int U = 8 / KM;        // tokens whose loads are in flight together
    constexpr int MW = 64 / KM;      // tokens per routing window
    __shared__ u32x4 wrt[NC * 64];   // [column][lane]: 16 bytes per lane and column
    T* wrt_e = (T*)wrt;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slice = blockIdx.x % n_slices;
    const int i0 = slice * SW;
    // this lane's chunk of the row; lanes past the row read chunk 0 and store nothing, so
    // that the wave stays converged for its readlanes
    const bool live = slice * 64 + lane < vpr;
    const int c = live ? slice * 64 + lane : 0;

    const int tb = (blockIdx.x / n_slices) * tok_per_block;
    const int per_wave = (tok_per_block + 3) >> 2;
    const int w_lo = __builtin_amdgcn_readfirstlane(min(tb + wave * per_wave, ntok));
    const int w_hi = __builtin_amdgcn_readfirstlane(min(tb + min((wave + 1) * per_wave, tok_per_block), ntok));
    // routing entries of a window: slot k of token tw + lane / KM (row -1 when dropped)
    int rv = -1, ev = 0;
    float wv = 0.f, zv = 0.f;
    auto load_window = [&](int tw) {
        const int my_t = tw + lane / KM, my_k = lane % KM;
        const bool slot = my_t < w_hi && my_k < K;
        const int64_t sk = (int64_t)my_t * K + my_k;
        rv = slot ? row_of[sk] : -1;
        ev = 0;
        wv = 0.f;
        if (dlogits && slot) {
            ev = topk_idx[sk];
            wv = dlogits[(int64_t)my_t * E + ev];
        }
        zv = dz && lane < MW && tw + lane < w_hi ? dz[tw + lane] : 0.f;
    };
    // the first window's entries are requested before the weight slice is staged, so that
    // the two loads overlap
    if (w_lo < w_hi) load_window(w_lo);

    // router weight slice: element (i, e) of w_router[d][E] -> wrt_e[e * SW + i - i0]
    if (dlogits) {
        if ((E % N) == 0) {
            // 16-byte loads: N consecutive experts of one row i
            const int per_row = E / N;
            const u32x4* src = (const u32x4*)(w_router + (int64_t)i0 * E);
            for (int q = threadIdx.x; q < SW * per_row; q += 256) {
                const int i = q / per_row, e0 = (q - i * per_row) * N;
                if (i0 + i < d) {
                    const u32x4 v = src[q];
                    const T* pv = (const T*)&v;
#pragma unroll
                    for (int j = 0; j < N; ++j) wrt_e[(e0 + j) * SW + i] = pv[j];
                } else {
#pragma unroll
                    for (int j = 0; j < N; ++j) wrt_e[(e0 + j) * SW + i] = T(0);
                }
            }
        } else {
            for (int idx = threadIdx.x; idx < SW * E; idx += 256) {
                const int i = idx / E, e = idx - i * E;
                wrt_e[e * SW + i] = i0 + i < d ? w_router[(int64_t)(i0 + i) * E + e] : T(0);
            }
        }
    }
    if (dz) {
        for (int i = threadIdx.x; i < SW; i += 256) wrt_e[E * SW + i] = i0 + i < d ? w_sg[i0 + i] : T(0);
    }
    __syncthreads();

    for (int tw = w_lo; tw < w_hi; tw += MW) {
        if (tw != w_lo) load_window(tw);
        const int wn = min(MW, w_hi - tw);
        for (int u0 = 0; u0 < wn; u0 += U) {
            u32x4 v[U][KM], va[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u0 + u >= wn) break;
                const int64_t t = tw + u0 + u;
#pragma unroll
                for (int k = 0; k < KM; ++k) {
                    const int row = __builtin_amdgcn_readlane(rv, (u0 + u) * KM + k);
                    if (row >= 0) v[u][k] = dxp[(int64_t)row * vpr + c];
                }
                if (dx_add) va[u] = dx_add[t * vpr + c];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u0 + u >= wn) break;
                const int64_t t = tw + u0 + u;
                float acc[N], f[N];
#pragma unroll
                for (int i = 0; i < N; ++i) acc[i] = 0.f;
#pragma unroll
                for (int k = 0; k < KM; ++k) {
                    const int row = __builtin_amdgcn_readlane(rv, (u0 + u) * KM + k);
                    if (row >= 0) {
                        Vec16<T>::unpack(v[u][k], f);
#pragma unroll
                        for (int i = 0; i < N; ++i) acc[i] += 1.0f * f[i];
                    }
                }
                if (dlogits) {
#pragma unroll
                    for (int k = 0; k < KM; ++k) {
                        if (k >= K) break;
                        const int sl = (u0 + u) * KM + k;
                        const int e = __builtin_amdgcn_readlane(ev, sl);
                        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), sl));
                        Vec16<T>::unpack(wrt[e * 64 + lane], f);
#pragma unroll
                        for (int i = 0; i < N; ++i) acc[i] += w * f[i];
                    }
                }
                if (dz) {
                    const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zv), u0 + u));
                    Vec16<T>::unpack(wrt[E * 64 + lane], f);
#pragma unroll
                    for (int i = 0; i < N; ++i) acc[i] += w * f[i];
                }
                if (dx_add) {
                    Vec16<T>::unpack(va[u], f);
#pragma unroll
                    for (int i = 0; i < N; ++i) acc[i] += 1.0f * f[i];
                }
                if (live) dx[t * vpr + c] = Vec16<T>::pack(acc);
            }
        }
    }
}

// dl for the K chosen experts: g_j (dgate_j - sum_k g_k dgate_k); 0 elsewhere.  The
// difference cancels when one gate is close to 1 (dgate_j - g_j dgate_j - ...), so it is
// formed in fp64: the products of two fp32 values are exact there, and dl is then
// correct to its own fp32 rounding (in fp32 the difference kept an absolute error of
// about one ulp of dgate_j, a relative error of up to 1e-4 on dl at g_j near 1).  K
// values per token: the fp64 cost is negligible.
__global__ void __launch_bounds__(256) dlogits_kernel(const int32_t* __restrict__ topk_idx,
                                                      const float* __restrict__ gate,
                                                      const float* __restrict__ dgate, int T,
                                                      int E, int K, float* __restrict__ dl) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    double inner = 0.0;
    for (int k = 0; k < K; ++k) inner += (double)gate[t * K + k] * (double)dgate[t * K + k];
    float v = 0.f;
    for (int k = 0; k < K; ++k)
        if (topk_idx[t * K + k] == lane)
            v = (float)((double)gate[t * K + k] * ((double)dgate[t * K + k] - inner));
    if (lane < E) dl[t * E + lane] = v;
}

// partial[c][i][e] = sum over tokens t of chunk c of x[t][i] * dcol[t][e], where the
// columns are dl (e < E) and dz (e == E).  A wave owns 8 consecutive i (one 16-byte
// x vector per lane... one per token) and 8 columns; chunks are summed in order later.
template <typename T>
__global__ void __launch_bounds__(256) router_wgrad_partial(
    const T* __restrict__ x, const float* __restrict__ dl, const float* __restrict__ dz, int T_,
    int d, int E, int ncol, int chunk, float* __restrict__ partial) {
    constexpr int N = Vec16<T>::N;       // i per lane
    constexpr int U = 8;                 // tokens whose loads are in flight together
    // waves 1..3 hand their sums to wave 0, lane-major (conflict-free)
    __shared__ float red[3][N * 8][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i0 = (blockIdx.x * 64 + lane) * N;
    const int c = blockIdx.y;
    const int e0 = blockIdx.z * 8;
    float acc[N][8];
#pragma unroll
    for (int a = 0; a < N; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = 0.f;
    const bool ok = i0 < d;
    // wave w sums the w-th quarter of the chunk's tokens
    // (wave-uniform bounds: the per-token dl and dz values are then scalar loads)
    const int sub = (chunk + 3) / 4;
    const int64_t cend = min((int64_t)(c + 1) * chunk, (int64_t)T_);
    const int64_t tb = __builtin_amdgcn_readfirstlane((int)((int64_t)c * chunk + (int64_t)wave * sub));
    const int64_t te = __builtin_amdgcn_readfirstlane((int)min(tb + sub, cend));
    for (int64_t t = tb; t < te; t += U) {
        // issue the loads of U tokens, then their FMAs
        u32x4 xr[U];
        float w[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t tt = t + u;
            const bool in = tt < te;
            xr[u] = (ok && in) ? *(const u32x4*)(x + tt * d + i0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int e = e0 + b;
                w[u][b] = !in ? 0.f : (e < E) ? dl[tt * E + e] : ((e == E && dz) ? dz[tt] : 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float xv[N];
            Vec16<T>::unpack(xr[u], xv);
#pragma unroll
            for (int a = 0; a < N; ++a)
#pragma unroll
                for (int b = 0; b < 8; ++b) acc[a][b] += xv[a] * w[u][b];
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int a = 0; a < N; ++a)
#pragma unroll
            for (int b = 0; b < 8; ++b) red[wave - 1][a * 8 + b][lane] = acc[a][b];
    }
    __syncthreads();
    if (wave == 0 && ok) {
        const int ncol8 = (ncol + 7) / 8 * 8;
#pragma unroll
        for (int a = 0; a < N; ++a)
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                float v = acc[a][b];
#pragma unroll
                for (int w = 0; w < 3; ++w) v += red[w][a * 8 + b][lane];  // fixed order
                partial[((int64_t)c * d + i0 + a) * ncol8 + e0 + b] = v;
            }
    }
}

// The same partial sums for many columns (E = 16, 32 or 64, + the shared gate) on the
// fp32 matrix cores: per chunk the partial is the product x_c^T dcol_c (K = the chunk's
// tokens), so a block stages the chunk's x rows for 256 consecutive i (16-byte loads) and
// its dl/dz columns (zero-padded to a multiple of 16) in LDS, and wave w accumulates
// i = i0 + 64w .. +63 against every column with v_mfma_f32_16x16x4_f32, four tokens per
// instruction, tokens in order.  x is read once whatever the number of columns, and the
// products and sums stay in fp32.
constexpr int RW_I = 256;      // i per block
constexpr int RW_TOK = 64;     // tokens per chunk (at most)
constexpr int RW_CT = 5;       // 16-column tiles: up to 80 columns

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T, int CT>
__global__ void __launch_bounds__(256) router_wgrad_partial_wide(
    const T* __restrict__ x, const float* __restrict__ dl, const float* __restrict__ dz, int T_,
    int d, int E, int ncol, int chunk, float* __restrict__ partial) {
    __shared__ __attribute__((aligned(16))) T sx[RW_TOK][RW_I];
    __shared__ float sw[RW_TOK][CT * 16];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int i0 = blockIdx.x * RW_I;
    const int c = blockIdx.y;
    const int64_t tb = (int64_t)c * chunk;
    const int nt = (int)min((int64_t)chunk, (int64_t)T_ - tb);
    const int ni = min(RW_I, d - i0);
    // stage x[tb .. tb+nt)[i0 .. i0+ni) in 16-byte pieces (d % 8 == 0, so ni is a whole
    // number of pieces) and the columns; zeros past the ends
    constexpr int P16 = Elem<T>::per16;
    constexpr int CPT = RW_I / P16;
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    for (int q = tid; q < RW_TOK * CPT; q += 256) {
        const int t = q / CPT, ch = q % CPT;
        const bool ok = t < nt && ch * P16 < ni;
        const v4u v = *(const v4u*)(x + (ok ? (tb + t) * d + i0 + ch * P16 : 0));
        *(v4u*)&sx[t][ch * P16] = ok ? v : v4u{0u, 0u, 0u, 0u};
    }
    for (int q = tid; q < RW_TOK * CT * 16; q += 256) {
        const int t = q / (CT * 16), e = q % (CT * 16);
        float v = 0.f;
        if (t < nt) v = e < E ? dl[(tb + t) * E + e] : (e == E && dz ? dz[tb + t] : 0.f);
        sw[t][e] = v;
    }
    __syncthreads();
    // A = x^T (16 i x 4 tokens): lane supplies x[t0 + lane/16][i]; B = dcol (4 tokens x 16
    // columns): lane supplies dcol[t0 + lane/16][col]; D: lane holds rows 4*(lane/16) + r,
    // column lane%16.
    f32x4_t acc[4][CT];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < CT; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int kr = lane >> 4, cc = lane & 15;
    for (int t0 = 0; t0 < RW_TOK; t0 += 4) {
        float av[4], bv[CT];
#pragma unroll
        for (int a = 0; a < 4; ++a) av[a] = Elem<T>::load(&sx[t0 + kr][0], wave * 64 + a * 16 + cc);
#pragma unroll
        for (int b = 0; b < CT; ++b) bv[b] = sw[t0 + kr][b * 16 + cc];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < CT; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    const int ncol8 = (ncol + 7) / 8 * 8;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int il = wave * 64 + a * 16 + 4 * kr + r;
            if (il >= ni) continue;
            float* out = partial + ((int64_t)c * d + i0 + il) * ncol8;
#pragma unroll
            for (int b = 0; b < CT; ++b) {
                const int e = b * 16 + cc;
                if (e < ncol) out[e] = acc[a][b][r];
            }
        }
}

// bf16 layers: partial[c][i][e] = sum over the tokens t of chunk c (RG_CHUNK tokens) of
// x[t][i] * dcol[t][e], on the bf16 matrix cores.  dcol (fp32) is split into two bf16
// terms, hi = bf16(v) and lo = bf16(v - hi), whose sum carries 16 significant bits (a
// relative error below 2^-17, far under the bf16 rounding of dW); x is bf16 already, so
// both products are exact and the MFMA accumulates them in fp32.  A block takes 128 i
// and one chunk, in k-steps of 32 tokens staged through LDS with two buffers: x as it
// is in memory ([32 t][128 i], 256-byte rows, 16-byte chunks XOR-swizzled, read as MFMA
// fragments with the LDS transpose read) and hi, lo transposed ([e][32 t], one 16-byte
// read per fragment).  Wave w owns i0 + 32 w .. +31 (two 16-row A tiles) and all CT
// 16-column tiles.
constexpr int RG_I = 128;
constexpr int RG_CHUNK = 512;
constexpr int RG_DEPTH = 4;    // register sets of the staging pipeline

typedef __bf16 rg_bf16x8 __attribute__((ext_vector_type(8)));
typedef short rg_s16x4 __attribute__((ext_vector_type(4)));
typedef short rg_s16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t rg_u32x4 __attribute__((ext_vector_type(4)));

// 16-byte chunk swizzle of a [32 t][128 i] tile: chunk p of row t holds logical chunk
// p ^ rg_swz(t); the transpose reads of a fragment (4 rows x 32 bytes per 16 lanes) then
// fall on distinct banks.
__device__ __forceinline__ int rg_swz(int t) { return (4 * (t & 3)) ^ (((t >> 3) & 1) << 1); }

template <int CT>
__global__ void __launch_bounds__(256) router_wgrad_mfma(const bf16_t* __restrict__ x,
                                                         const float* __restrict__ dl,
                                                         const float* __restrict__ dz, int T_,
                                                         int d, int E, int ncol,
                                                         float* __restrict__ partial) {
    constexpr int NC = CT * 16;       // columns, zero past ncol
    constexpr int PT = 40;            // row pitch (bf16) of the transposed hi, lo tiles
    constexpr int NPAIR = NC * 4;     // (column, 8-token group) pairs per k-step
    constexpr int PPT = (NPAIR + 255) / 256;
    __shared__ __attribute__((aligned(16))) char sx[2][32 * 256];
    __shared__ __attribute__((aligned(16))) bf16_t sh[2][NC][PT];
    __shared__ __attribute__((aligned(16))) bf16_t sl[2][NC][PT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int i0 = blockIdx.x * RG_I;
    const int64_t tb = (int64_t)blockIdx.y * RG_CHUNK;
    const int nt = (int)min((int64_t)RG_CHUNK, (int64_t)T_ - tb);
    const int nks = (nt + 31) / 32;

    // staging: x rows t = tid / 16 and t + 16, chunk tid % 16 (8 i); dcol pairs
    // p = tid + 256 j: column p / 4, tokens 8 (p % 4) .. +7.  The loads of a k-step go into
    // one of RG_DEPTH register sets, RG_DEPTH - 1 k-steps ahead of its LDS stores.
    const int xt = tid >> 4, xch = tid & 15;
    const bool x_ok = i0 + 8 * xch < d;  // d % 8 == 0: a chunk is wholly in or out
    const bf16_t* xs = x + tb * d + (x_ok ? i0 + 8 * xch : 0);
    // column source of each pair: dl (stride E), dz (stride 1), or none (reads dl, zeroed)
    const float* csrc[PPT];
    int cstride[PPT];
    bool clive[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int p = tid + 256 * j;
        const int e = p >> 2;
        const bool in = p < NPAIR;
        const bool from_dz = in && e == E && dz;
        clive[j] = in && (e < E || from_dz);
        csrc[j] = from_dz ? dz + tb : dl + tb * E + (in && e < E ? e : 0);
        cstride[j] = from_dz ? 1 : E;
    }
    // Every load is issued unconditionally from a valid address (tokens past the chunk read
    // its last token); values that do not exist are zeroed when they are stored to LDS.
    struct Regs {
        u32x4 x[2];
        float c[PPT][8];
    };
    auto load_regs = [&](Regs& R, int ks) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int tl = min(32 * ks + xt + 16 * h, nt - 1);
            R.x[h] = *(const u32x4*)(xs + (int64_t)tl * d);
        }
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int tg = (tid + 256 * j) & 3;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int tl = min(32 * ks + 8 * tg + u, nt - 1);
                R.c[j][u] = csrc[j][(int64_t)tl * cstride[j]];
            }
        }
    };
    auto store_lds = [&](const Regs& R, int ks, int b) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int t = xt + 16 * h;
            const bool ok = x_ok && 32 * ks + t < nt;
            *(u32x4*)(sx[b] + t * 256 + ((xch ^ rg_swz(t)) << 4)) = ok ? R.x[h] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int p = tid + 256 * j;
            if (p < NPAIR) {
                const int e = p >> 2, tg = p & 3;
                float hi[8], lo[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float v = (clive[j] && 32 * ks + 8 * tg + u < nt) ? R.c[j][u] : 0.f;
                    hi[u] = bf16_to_f32(f32_to_bf16(v));
                    lo[u] = v - hi[u];
                }
                *(u32x4*)&sh[b][e][8 * tg] = Vec16<bf16_t>::pack(hi);
                *(u32x4*)&sl[b][e][8 * tg] = Vec16<bf16_t>::pack(lo);
            }
        }
    };

    f32x4_t acc[2][CT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // fragment addresses: A (x^T, rows i) by the transpose read of 4 rows x 8 bytes per
    // 16 lanes (lane s of group g: k row 8 g + s / 4, columns 4 (s % 4) .. +3; the second
    // read 4 k rows further); B (hi, lo) one 16-byte read of 8 tokens of column lane % 16
    const int g = lane >> 4, sl16 = lane & 15;
    uint32_t a_off[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int col = 32 * wave + 16 * a + 4 * (sl16 & 3);
        const int kr = 8 * g + (sl16 >> 2);
        a_off[a] = kr * 256 + (((col >> 3) ^ rg_swz(kr)) << 4) + (col & 7) * 2;
    }
    auto compute = [&](int b) {
        typedef __attribute__((address_space(3))) rg_s16x4 lds_s16x4;
        rg_bf16x8 af[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(sx[b]) + a_off[a];
            const rg_s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)base);
            const rg_s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(base + 1024));
            const rg_s16x8 v = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            af[a] = __builtin_bit_cast(rg_bf16x8, v);
        }
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const rg_bf16x8 bh = __builtin_bit_cast(rg_bf16x8, *(const rg_u32x4*)&sh[b][16 * c + sl16][8 * g]);
            const rg_bf16x8 bl = __builtin_bit_cast(rg_bf16x8, *(const rg_u32x4*)&sl[b][16 * c + sl16][8 * g]);
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bh, acc[a][c], 0, 0, 0);
                acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bl, acc[a][c], 0, 0, 0);
            }
        }
    };

    // Loads run RG_DEPTH - 1 k-steps ahead; near the chunk's end they repeat its last
    // k-step (unused), so that they are issued unconditionally.  LDS buffer ks & 1 is
    // written after the barrier that ends the compute of k-step ks - 2.
    Regs R[RG_DEPTH];
    if (nks > 0) {
#pragma unroll
        for (int j = 0; j < RG_DEPTH - 1; ++j) load_regs(R[j], min(j, nks - 1));
    }
    for (int ks0 = 0; ks0 < nks; ks0 += RG_DEPTH) {
#pragma unroll
        for (int u = 0; u < RG_DEPTH; ++u) {
            const int ks = ks0 + u;
            if (ks >= nks) break;
            load_regs(R[(u + RG_DEPTH - 1) % RG_DEPTH], min(ks + RG_DEPTH - 1, nks - 1));
            store_lds(R[u], ks, ks & 1);
            __syncthreads();
            compute(ks & 1);
        }
    }
    // D of the 16x16 MFMA: lane holds column e = 16 c + lane % 16 and rows
    // i = 4 (lane / 16) + r of the A tile
    const int ncol8 = (ncol + 7) / 8 * 8;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 32 * wave + 16 * a + 4 * g + r;
            if (i >= d) continue;
            float* out = partial + ((int64_t)blockIdx.y * d + i) * ncol8;
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const int e = 16 * c + sl16;
                if (e < ncol) out[e] = acc[a][c][r];
            }
        }
}

template <typename T>
__global__ void __launch_bounds__(256) router_wgrad_final(const float* __restrict__ partial,
                                                          int n_chunks, int d, int E, int ncol,
                                                          T* __restrict__ dw, T* __restrict__ dw_sg) {
    int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int ncol8 = (ncol + 7) / 8 * 8;
    if (idx >= (int64_t)d * ncol) return;
    int i = (int)(idx / ncol), e = (int)(idx % ncol);
    float s = 0.f;
#pragma unroll 8
    for (int c = 0; c < n_chunks; ++c) s += partial[((int64_t)c * d + i) * ncol8 + e];
    if (e < E) Elem<T>::store(dw, (int64_t)i * E + e, s);
    else Elem<T>::store(dw_sg, i, s);
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_permute(const moe_desc& d, int64_t R, const void* x, const moe_routing& r,
                          void* xp, hipStream_t s) {
    const int esz = d.dtype == MOE_BF16 ? 2 : 4;
    const int vpr = d.d * esz / 16;
    if (R > 0 && d.T > 0) {
        const unsigned nb = blocks_for(d.T, ROWS_PER_BLOCK);
        auto go = [&](auto km) {
            permute_kernel<decltype(km)::value><<<nb, 256, 0, s>>>(
                (const u32x4*)x, r.row_of, d.T, d.K, vpr, (u32x4*)xp);
        };
        if (d.K <= 2) go(std::integral_constant<int, 2>{});
        else if (d.K <= 4) go(std::integral_constant<int, 4>{});
        else go(std::integral_constant<int, 8>{});
    }
    return hipGetLastError();
}

// Runs go(T{}, std::integral_constant<int, KM>{}) with the element type of the layer and
// the smallest slot bound KM in {2, 4, 8} that covers K.
template <typename F>
void by_dtype_and_slots(const moe_desc& d, F&& go) {
    auto by_k = [&](auto tag) {
        if (d.K <= 2) go(tag, std::integral_constant<int, 2>{});
        else if (d.K <= 4) go(tag, std::integral_constant<int, 4>{});
        else go(tag, std::integral_constant<int, 8>{});
    };
    if (d.dtype == MOE_BF16) by_k(bf16_t{});
    else by_k(float{});
}

hipError_t launch_unpermute(const moe_desc& d, const void* o, const moe_routing& r,
                            const void* shared, const float* z, void* y, hipStream_t s) {
    const int esz = d.dtype == MOE_BF16 ? 2 : 4;
    const int vpr = d.d * esz / 16;
    const unsigned nb = blocks_for(d.T, ROWS_PER_BLOCK);
    by_dtype_and_slots(d, [&](auto tag, auto km) {
        using T = decltype(tag);
        unpermute_kernel<T, decltype(km)::value><<<nb, 256, 0, s>>>(
            (const u32x4*)o, r.row_of, r.topk_gate, (const u32x4*)shared, z, d.T, d.K, vpr,
            (u32x4*)y);
    });
    return hipGetLastError();
}

hipError_t launch_unpermute_bwd(const moe_desc& d, const void* dy, const void* o,
                                const moe_routing& r, const void* shared, const float* z,
                                void* d_o, float* dgate, void* dshared, float* dz, hipStream_t s) {
    const int esz = d.dtype == MOE_BF16 ? 2 : 4;
    const int vpr = d.d * esz / 16;
    const unsigned nb = blocks_for(d.T, ROWS_PER_BLOCK);
    by_dtype_and_slots(d, [&](auto tag, auto km) {
        using T = decltype(tag);
        unpermute_bwd_kernel<T, decltype(km)::value><<<nb, 256, 0, s>>>(
            (const u32x4*)dy, (const u32x4*)o, r.row_of, r.topk_gate, (const u32x4*)shared, z, d.T,
            d.K, vpr, (u32x4*)d_o, dgate, (u32x4*)dshared, dz);
    });
    return hipGetLastError();
}

hipError_t launch_permute_bwd(const moe_desc& d, const void* dxp, const moe_routing& r,
                              const float* dlogits, const void* w_router, const float* dz,
                              const void* w_sg, const void* dx_add, void* dx, void* w_rt,
                              hipStream_t s) {
    if (d.T == 0) return hipSuccess;
    const int esz = d.dtype == MOE_BF16 ? 2 : 4;
    const int vpr = d.d * esz / 16;
    const int ncol = d.E + 1;  // router columns and w_sg
    if (ncol > kPermuteBwdSliceCols) {
        // many experts: transposed weight rows in the workspace, one wave per token
        const bool need_rt = dlogits || dz;
        const unsigned nb = blocks_for(d.T, ROWS_PER_BLOCK);
        const unsigned tb = blocks_for((int64_t)ncol * d.d, 256);
        by_dtype_and_slots(d, [&](auto tag, auto km) {
            using T = decltype(tag);
            if (need_rt)
                transpose_rw_kernel<T><<<tb, 256, 0, s>>>((const T*)w_router, (const T*)w_sg,
                                                          (T*)w_rt, d.d, d.E, ncol);
            permute_bwd_rows_kernel<T, decltype(km)::value><<<nb, 256, 0, s>>>(
                (const u32x4*)dxp, r.row_of, r.topk_idx, dlogits, (const u32x4*)w_rt, dz,
                (const u32x4*)dx_add, d.T, d.E, d.K, vpr, (u32x4*)dx);
        });
        return hipGetLastError();
    }
    const int n_slices = (vpr + 63) / 64;
    const int tpb = 32;  // tokens per block (8 per wave): measured best of 16-256
    const int64_t nb = (int64_t)n_slices * ((d.T + tpb - 1) / tpb);
    if (nb > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    auto go = [&](auto tag, auto km) {
        using T = decltype(tag);
        permute_bwd_kernel<T, decltype(km)::value, kPermuteBwdSliceCols><<<(unsigned)nb, 256, 0, s>>>(
            (const u32x4*)dxp, r.row_of, r.keep, r.topk_idx, dlogits, (const T*)w_router, dz,
            (const T*)w_sg, (const u32x4*)dx_add, d.T, d.d, d.E, d.K, vpr, n_slices, tpb,
            (u32x4*)dx);
    };
    using K2 = std::integral_constant<int, 2>;
    using K8 = std::integral_constant<int, 8>;
    auto by_k = [&](auto tag) {
        if (d.K <= 2) go(tag, K2{});
        else go(tag, K8{});
    };
    if (d.dtype == MOE_BF16) by_k(bf16_t{});
    else by_k(float{});
    return hipGetLastError();
}

int router_bwd_chunk(int dtype) { return dtype == MOE_BF16 ? RG_CHUNK : RW_TOK; }

hipError_t launch_router_bwd(const moe_desc& d, const void* x, const moe_routing& r,
                             const float* dgate, const float* dz, float* dlogits, void* dw_router,
                             void* dw_sg, float* partial, int n_chunks, int chunk, hipStream_t s) {
    const int ncol = d.E + (dz ? 1 : 0);
    const int per = d.dtype == MOE_BF16 ? 8 : 4;
    dim3 g1(blocks_for(d.d / per, 64), n_chunks, (ncol + 7) / 8);
    const unsigned g2 = blocks_for((int64_t)d.d * ncol, 256);
    if (d.T > 0)  // with no token the final pass alone writes zero gradients
        dlogits_kernel<<<blocks_for(d.T, 4), 256, 0, s>>>(r.topk_idx, r.topk_gate, dgate, d.T,
                                                           d.E, d.K, dlogits);
    // many columns: the matrix-core kernel (chunks of at most RW_TOK tokens)
    const int ct = (ncol + 15) / 16;
    const bool wide = ncol > 8 && ct <= RW_CT && chunk <= RW_TOK && n_chunks > 0;
    const dim3 gw(blocks_for(d.d, RW_I), n_chunks);
    auto launch_wide = [&](auto tag) {
        using T = decltype(tag);
        const T* xt = (const T*)x;
        if (ct <= 1)
            router_wgrad_partial_wide<T, 1><<<gw, 256, 0, s>>>(xt, dlogits, dz, d.T, d.d, d.E, ncol, chunk, partial);
        else if (ct <= 2)
            router_wgrad_partial_wide<T, 2><<<gw, 256, 0, s>>>(xt, dlogits, dz, d.T, d.d, d.E, ncol, chunk, partial);
        else if (ct <= 3)
            router_wgrad_partial_wide<T, 3><<<gw, 256, 0, s>>>(xt, dlogits, dz, d.T, d.d, d.E, ncol, chunk, partial);
        else if (ct <= 4)
            router_wgrad_partial_wide<T, 4><<<gw, 256, 0, s>>>(xt, dlogits, dz, d.T, d.d, d.E, ncol, chunk, partial);
        else
            router_wgrad_partial_wide<T, 5><<<gw, 256, 0, s>>>(xt, dlogits, dz, d.T, d.d, d.E, ncol, chunk, partial);
    };
    if (d.dtype == MOE_BF16) {
        // chunks of RG_CHUNK tokens on the bf16 matrix cores
        if (chunk != RG_CHUNK || ct > RW_CT) return hipErrorInvalidValue;
        const dim3 gm(blocks_for(d.d, RG_I), n_chunks);
        const bf16_t* xb = (const bf16_t*)x;
        if (n_chunks > 0) {
            switch (ct) {
                case 1: router_wgrad_mfma<1><<<gm, 256, 0, s>>>(xb, dlogits, dz, d.T, d.d, d.E, ncol, partial); break;
                case 2: router_wgrad_mfma<2><<<gm, 256, 0, s>>>(xb, dlogits, dz, d.T, d.d, d.E, ncol, partial); break;
                case 3: router_wgrad_mfma<3><<<gm, 256, 0, s>>>(xb, dlogits, dz, d.T, d.d, d.E, ncol, partial); break;
                case 4: router_wgrad_mfma<4><<<gm, 256, 0, s>>>(xb, dlogits, dz, d.T, d.d, d.E, ncol, partial); break;
                default: router_wgrad_mfma<5><<<gm, 256, 0, s>>>(xb, dlogits, dz, d.T, d.d, d.E, ncol, partial); break;
            }
        }
        router_wgrad_final<bf16_t><<<g2, 256, 0, s>>>(partial, n_chunks, d.d, d.E, ncol,
                                                       (bf16_t*)dw_router, (bf16_t*)dw_sg);
    } else {
        if (wide)
            launch_wide(float{});
        else if (n_chunks > 0)
            router_wgrad_partial<float><<<g1, 256, 0, s>>>((const float*)x, dlogits, dz, d.T, d.d,
                                                           d.E, ncol, chunk, partial);
        router_wgrad_final<float><<<g2, 256, 0, s>>>(partial, n_chunks, d.d, d.E, ncol,
                                                      (float*)dw_router, (float*)dw_sg);
    }
    return hipGetLastError();
}

}  // namespace moe
