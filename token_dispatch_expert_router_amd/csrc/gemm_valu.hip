// Grouped GEMMs of the SwiGLU experts on the vector ALUs: the fp32 path, and the bf16
// path for shapes the matrix-core kernel does not tile (d or f not a multiple of 256).
// Same six passes and the same segment decoding as the MFMA kernel ("MoE Parallel
// Folding", arXiv 2504.14960, knowledge-base notes page, method paragraph: expert FFN
// computation on the permuted, expert-contiguous rows), with 64 x 64 tiles, k-step
// 16, 256 threads each computing 4 x 4 outputs from LDS, fp32 accumulation and
// bounds checks on every operand access.
#include "common.h"

namespace moe {
namespace {

constexpr int VB = 64;   // tile edge
constexpr int VK = 16;   // k-step

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
    return Elem<T>::load((const T*)p, i);
}
template <typename T>
__device__ __forceinline__ void st(void* p, int64_t i, float v) {
    Elem<T>::store((T*)p, i, v);
}

template <typename T, int MODE>
__global__ void __launch_bounds__(256) gg_valu_kernel(GemmArgs g) {
    __shared__ float As[VK][VB + 1];
    __shared__ float Bs[VK][VB + 1];
    __shared__ float Bu[VK][VB + 1];  // up projection (gate/up pass only)
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int L = blockIdx.x;
    const int d = g.d, f = g.f;

    int e = 0, m0 = 0, m_lim = 0, n0 = 0, N = 0, M_out = 0, K = 0, k_lo = 0;
    if (MODE <= GG_DGRAD_GATEUP) {
        N = (MODE == GG_FWD_GATEUP || MODE == GG_DGRAD_DOWN) ? f : d;
        const int n_tiles = (N + VB - 1) / VB;
        int acc = 0;
        bool found = false;
        for (int i = 0; i < g.E && !found; ++i) {
            const int lo = g.offsets[i], hi = g.offsets[i + 1];
            const int mt = (hi - lo + VB - 1) / VB;
            if (L < acc + mt * n_tiles) {
                const int loc = L - acc;
                e = i;
                m0 = lo + (loc % mt) * VB;
                m_lim = hi;
                n0 = (loc / mt) * VB;
                found = true;
            }
            acc += mt * n_tiles;
        }
        if (!found) return;
        K = MODE == GG_FWD_GATEUP ? d : MODE == GG_FWD_DOWN ? f : MODE == GG_DGRAD_DOWN ? d : 2 * f;
    } else {
        M_out = MODE == GG_WGRAD_DOWN ? f : d;
        N = MODE == GG_WGRAD_DOWN ? d : 2 * f;
        const int MT = (M_out + VB - 1) / VB, NTl = (N + VB - 1) / VB;
        e = L / (MT * NTl);
        if (e >= g.E) return;
        const int loc = L - e * MT * NTl;
        m0 = (loc % MT) * VB;
        n0 = (loc / MT) * VB;
        m_lim = M_out;
        k_lo = g.offsets[e];
        K = g.offsets[e + 1] - k_lo;
    }

    // A(m, k) and B(k, n) of this pass (0 outside the operand).
    auto A = [&](int m, int k) -> float {
        if (m >= m_lim || k >= K) return 0.f;
        switch (MODE) {
            case GG_FWD_GATEUP: return ld<T>(g.A0, (int64_t)m * d + k);
            case GG_FWD_DOWN: return ld<T>(g.A0, (int64_t)m * f + k);
            case GG_DGRAD_DOWN: return ld<T>(g.A0, (int64_t)m * d + k);
            case GG_DGRAD_GATEUP:
                return k < f ? ld<T>(g.A0, (int64_t)m * f + k) : ld<T>(g.A1, (int64_t)m * f + k - f);
            case GG_WGRAD_DOWN: return ld<T>(g.A0, (int64_t)(k_lo + k) * f + m);
            default: return ld<T>(g.A0, (int64_t)(k_lo + k) * d + m);
        }
    };
    auto B = [&](int k, int n) -> float {
        if (n >= N || k >= K) return 0.f;
        switch (MODE) {
            case GG_FWD_GATEUP: return ld<T>(g.B0, (int64_t)e * d * f + (int64_t)k * f + n);
            case GG_FWD_DOWN: return ld<T>(g.B0, (int64_t)e * f * d + (int64_t)k * d + n);
            case GG_DGRAD_DOWN: return ld<T>(g.B0, (int64_t)e * f * d + (int64_t)n * d + k);
            case GG_DGRAD_GATEUP:
                return k < f ? ld<T>(g.B0, (int64_t)e * d * f + (int64_t)n * f + k)
                             : ld<T>(g.B1, (int64_t)e * d * f + (int64_t)n * f + k - f);
            case GG_WGRAD_DOWN: return ld<T>(g.B0, (int64_t)(k_lo + k) * d + n);
            default:
                return n < f ? ld<T>(g.B0, (int64_t)(k_lo + k) * f + n)
                             : ld<T>(g.B1, (int64_t)(k_lo + k) * f + n - f);
        }
    };

    float acc[4][4], accu[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) { acc[i][j] = 0.f; accu[i][j] = 0.f; }

    for (int k0 = 0; k0 < K; k0 += VK) {
        for (int idx = tid; idx < VK * VB; idx += 256) {
            const int kk = idx / VB, mm = idx % VB;
            As[kk][mm] = A(m0 + mm, k0 + kk);
            Bs[kk][mm] = B(k0 + kk, n0 + mm);
            if (MODE == GG_FWD_GATEUP) {
                const int n = n0 + mm, k = k0 + kk;
                Bu[kk][mm] = (n < N && k < K)
                                 ? ld<T>(g.B1, (int64_t)e * d * f + (int64_t)k * f + n) : 0.f;
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < VK; ++kk) {
            float a[4], b[4], bu[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b[j] = Bs[kk][tx * 4 + j];
                bu[j] = MODE == GG_FWD_GATEUP ? Bu[kk][tx * 4 + j] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] += a[i] * b[j];
                    if (MODE == GG_FWD_GATEUP) accu[i][j] += a[i] * bu[j];
                }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= m_lim) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            const float v = acc[i][j];
            if (MODE == GG_FWD_GATEUP) {
                const float b = accu[i][j];
                const int64_t o = (int64_t)m * f + n;
                st<T>(g.C0, o, v);
                st<T>(g.C1, o, b);
                st<T>(g.C2, o, v / (1.0f + __expf(-v)) * b);
            } else if (MODE == GG_FWD_DOWN || MODE == GG_DGRAD_GATEUP) {
                if (g.out_f32) ((float*)g.C0)[(int64_t)m * d + n] = v;
                else st<T>(g.C0, (int64_t)m * d + n, v);
            } else if (MODE == GG_DGRAD_DOWN) {
                const int64_t o = (int64_t)m * f + n;
                const float a = ld<T>(g.X0, o), b = ld<T>(g.X1, o);
                const float sg = 1.0f / (1.0f + __expf(-a));
                st<T>(g.C0, o, v * b * sg * (1.0f + a * (1.0f - sg)));
                st<T>(g.C1, o, v * a * sg);
            } else if (MODE == GG_WGRAD_DOWN) {
                st<T>(g.C0, (int64_t)e * f * d + (int64_t)m * d + n, v);
            } else {
                if (n < f) st<T>(g.C0, (int64_t)e * d * f + (int64_t)m * f + n, v);
                else st<T>(g.C1, (int64_t)e * d * f + (int64_t)m * f + n - f, v);
            }
        }
    }
}

template <typename T>
hipError_t launch_typed(GemmMode mode, const GemmArgs& a, hipStream_t s) {
    const int64_t mt_max = (a.R + VB - 1) / VB + a.E;
    auto ct = [](int64_t v) { return (v + VB - 1) / VB; };
    int64_t tiles;
    switch (mode) {
        case GG_FWD_GATEUP: tiles = mt_max * ct(a.f); break;
        case GG_FWD_DOWN: tiles = mt_max * ct(a.d); break;
        case GG_DGRAD_DOWN: tiles = mt_max * ct(a.f); break;
        case GG_DGRAD_GATEUP: tiles = mt_max * ct(a.d); break;
        case GG_WGRAD_DOWN: tiles = a.E * ct(a.f) * ct(a.d); break;
        default: tiles = a.E * ct(a.d) * ct(2 * (int64_t)a.f); break;
    }
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const unsigned nb = (unsigned)tiles;
    switch (mode) {
        case GG_FWD_GATEUP: gg_valu_kernel<T, GG_FWD_GATEUP><<<nb, 256, 0, s>>>(a); break;
        case GG_FWD_DOWN: gg_valu_kernel<T, GG_FWD_DOWN><<<nb, 256, 0, s>>>(a); break;
        case GG_DGRAD_DOWN: gg_valu_kernel<T, GG_DGRAD_DOWN><<<nb, 256, 0, s>>>(a); break;
        case GG_DGRAD_GATEUP: gg_valu_kernel<T, GG_DGRAD_GATEUP><<<nb, 256, 0, s>>>(a); break;
        case GG_WGRAD_DOWN: gg_valu_kernel<T, GG_WGRAD_DOWN><<<nb, 256, 0, s>>>(a); break;
        default: gg_valu_kernel<T, GG_WGRAD_GATEUP><<<nb, 256, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_valu(GemmMode mode, bool bf16, const GemmArgs& a, hipStream_t s) {
    return bf16 ? launch_typed<bf16_t>(mode, a, s) : launch_typed<float>(mode, a, s);
}

}  // namespace moe
