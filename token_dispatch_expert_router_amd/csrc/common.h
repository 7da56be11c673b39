// Shared device helpers of the MI355X MoE library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_WAVE 64

typedef uint16_t bf16_t;  // raw bfloat16 bits

// 16-byte vector used for every coalesced row access.
struct __attribute__((aligned(16))) u32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(((uint32_t)v) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
    static constexpr int per16 = 4;  // elements per 16 bytes
};
template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ float load(const bf16_t* p, int64_t i) {
        return bf16_to_f32(p[i]);
    }
    static __device__ __forceinline__ void store(bf16_t* p, int64_t i, float v) {
        p[i] = f32_to_bf16(v);
    }
    static constexpr int per16 = 8;
};

// Unpack 16 bytes into floats / pack floats into 16 bytes.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void unpack(const u32x4& v, float* o) {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
    static __device__ __forceinline__ u32x4 pack(const float* o) {
        u32x4 v;
        v.x = __float_as_uint(o[0]); v.y = __float_as_uint(o[1]);
        v.z = __float_as_uint(o[2]); v.w = __float_as_uint(o[3]);
        return v;
    }
};
template <> struct Vec16<bf16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void unpack(const u32x4& v, float* o) {
        o[0] = lo_bf16(v.x); o[1] = hi_bf16(v.x); o[2] = lo_bf16(v.y); o[3] = hi_bf16(v.y);
        o[4] = lo_bf16(v.z); o[5] = hi_bf16(v.z); o[6] = lo_bf16(v.w); o[7] = hi_bf16(v.w);
    }
    static __device__ __forceinline__ u32x4 pack(const float* o) {
        u32x4 v;
        v.x = pack_bf16x2(o[0], o[1]); v.y = pack_bf16x2(o[2], o[3]);
        v.z = pack_bf16x2(o[4], o[5]); v.w = pack_bf16x2(o[6], o[7]);
        return v;
    }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MOE_WAVE);
    return v;
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }
__device__ __forceinline__ float sigmoid_f(float a) { return 1.0f / (1.0f + __expf(-a)); }

// ---------------------------------------------------------------------------------
// Host-side launch helpers (declared here, defined in the .hip files).
// ---------------------------------------------------------------------------------
namespace moe {

struct RouteWs {
    int32_t* kcnt;  // [n_sub * E] kept per (sub-sequence, expert)
    int32_t* list;  // [n_sub * E * S] kept slots per group, token order
};

hipError_t launch_router_fwd(const moe_desc& d, const void* x, const void* w_router,
                             const float* bias, const void* w_sg, float* logits,
                             float* sg_logit, const moe_routing& r, hipStream_t s,
                             void* w_rt_ws);
hipError_t launch_topk_from_logits(const moe_desc& d, const float* logits,
                                   const moe_routing& r, hipStream_t s);
hipError_t launch_select_and_maps(const moe_desc& d, const moe_routing& r, RouteWs ws,
                                  hipStream_t s);

hipError_t launch_permute(const moe_desc& d, int64_t R, const void* x, const moe_routing& r,
                          void* xp, hipStream_t s);
hipError_t launch_unpermute(const moe_desc& d, const void* o, const moe_routing& r,
                            const void* shared, const float* sg_logit, void* y, hipStream_t s);
hipError_t launch_unpermute_bwd(const moe_desc& d, const void* dy, const void* o,
                                const moe_routing& r, const void* shared, const float* sg_logit,
                                void* d_o, float* dgate, void* dshared, float* dsg,
                                hipStream_t s);
hipError_t launch_permute_bwd(const moe_desc& d, const void* dxp, const moe_routing& r,
                              const float* dlogits, const void* w_router, const float* dsg,
                              const void* w_sg, const void* dx_add, void* dx, void* w_rt,
                              hipStream_t s);
// moe_permute_bwd keeps a block's slice of the router weight (E columns and w_sg) in LDS
// when E + 1 is at most this; more experts use a transposed copy in the workspace.
constexpr int kPermuteBwdSliceCols = 16;
// Tokens per partial sum of the router weight gradient (the workspace holds one
// d x ncol fp32 partial per chunk).
int router_bwd_chunk(int dtype);
hipError_t launch_router_bwd(const moe_desc& d, const void* x, const moe_routing& r,
                             const float* dgate, const float* dsg, float* dlogits,
                             void* dw_router, void* dw_sg, float* partial, int n_chunks,
                             int chunk, hipStream_t s);

// Grouped GEMM passes.
enum GemmMode {
    GG_FWD_GATEUP = 0,   // [a|b] = xp [W_g|W_u], h = silu(a) b
    GG_FWD_DOWN = 1,     // o = h W_d
    GG_DGRAD_DOWN = 2,   // dh = d_o W_d^T -> da, db
    GG_DGRAD_GATEUP = 3, // dxp = da W_g^T + db W_u^T
    GG_WGRAD_DOWN = 4,   // dW_d = h^T d_o
    GG_WGRAD_GATEUP = 5  // dW_g = xp^T da, dW_u = xp^T db
};

struct GemmArgs {
    int E, R, d, f;
    const int32_t* offsets;
    const void* A0;  // main row operand
    const void* A1;  // second half (dgrad gate/up: db)
    const void* B0;  // weights or second row operand
    const void* B1;
    const void* X0;  // epilogue inputs (a, b in dgrad down)
    const void* X1;
    void* C0;
    void* C1;
    void* C2;
    int out_f32;  // fwd down / dgrad gate/up: C0 is fp32 (partial sums over an f shard)
    int row_map;  // row passes: which XCD runs which tile (tiles::RowMap), set by the launcher
};

bool mfma_shape_ok(const moe_desc& d);
hipError_t launch_gemm_mfma(GemmMode mode, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_valu(GemmMode mode, bool bf16, const GemmArgs& a, hipStream_t s);

}  // namespace moe
