// C ABI of the MoE layer: host-side validation, workspace layout and launches.
// Every check happens before the first HIP call; a failed check launches nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "common.h"

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

moe_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define REQUIRE(cond, st, ...)                         \
    do {                                               \
        if (!(cond)) return fail((st), __VA_ARGS__);   \
    } while (0)

moe_status check_desc(const moe_desc* d) {
    REQUIRE(d, MOE_ERR_INVALID_ARG, "desc is NULL");
    REQUIRE(d->dtype == MOE_F32 || d->dtype == MOE_BF16, MOE_ERR_UNSUPPORTED,
            "dtype %d is not MOE_F32 or MOE_BF16", d->dtype);
    REQUIRE(d->T >= 0, MOE_ERR_INVALID_ARG, "T = %d < 0", d->T);
    REQUIRE(d->d > 0 && d->f > 0, MOE_ERR_INVALID_ARG, "d = %d and f = %d must be positive",
            d->d, d->f);
    REQUIRE(d->d % 8 == 0 && d->f % 8 == 0, MOE_ERR_UNSUPPORTED,
            "d = %d and f = %d must be multiples of 8", d->d, d->f);
    REQUIRE(d->E >= 1 && d->E <= 64, MOE_ERR_UNSUPPORTED, "E = %d outside [1, 64]", d->E);
    REQUIRE(d->K >= 1 && d->K <= d->E, MOE_ERR_INVALID_ARG, "K = %d outside [1, E = %d]", d->K,
            d->E);
    REQUIRE(d->K <= 8, MOE_ERR_UNSUPPORTED, "K = %d > 8", d->K);
    REQUIRE(d->sub_seq >= 1, MOE_ERR_INVALID_ARG, "sub_seq = %d < 1", d->sub_seq);
    REQUIRE(d->T % d->sub_seq == 0, MOE_ERR_INVALID_ARG, "T = %d is not a multiple of S = %d",
            d->T, d->sub_seq);
    REQUIRE(d->capacity >= -1, MOE_ERR_INVALID_ARG, "capacity = %d < -1", d->capacity);
    REQUIRE((int64_t)d->T * d->K < (int64_t)1 << 30, MOE_ERR_UNSUPPORTED, "T*K too large");
    REQUIRE((d->flags & ~(MOE_FLAG_VALU_GEMM | MOE_FLAG_F32_PARTIAL)) == 0, MOE_ERR_INVALID_ARG,
            "unknown flags 0x%x", d->flags);
    return MOE_OK;
}

// The row-movement calls read o and dxp in the layer's dtype; fp32 partial sums over an
// f shard are summed across shards (and cast) before they come back to them.
moe_status check_no_partial(const moe_desc& d, const char* fn) {
    REQUIRE(!(d.flags & MOE_FLAG_F32_PARTIAL), MOE_ERR_INVALID_ARG,
            "%s does not take MOE_FLAG_F32_PARTIAL (its row buffers are in the layer dtype)", fn);
    return MOE_OK;
}

// With T == 0 the per-token arrays are empty and may be NULL; the per-expert ones
// (kept_counts, offsets, n_kept) are always written.
moe_status check_routing(const moe_routing* r, int T) {
    REQUIRE(r, MOE_ERR_INVALID_ARG, "routing is NULL");
    REQUIRE(r->kept_counts && r->offsets && r->n_kept, MOE_ERR_INVALID_ARG,
            "a routing pointer is NULL");
    REQUIRE(T == 0 || (r->topk_idx && r->topk_prob && r->topk_gate && r->keep && r->row_of &&
                       r->src_of && r->routed_counts),
            MOE_ERR_INVALID_ARG, "a routing pointer is NULL");
    return MOE_OK;
}

int64_t max_rows(const moe_desc& d) {
    const int64_t tk = (int64_t)d.T * d.K;
    if (d.capacity < 0) return tk;
    const int64_t cap_rows = (int64_t)(d.T / d.sub_seq) * d.E * d.capacity;
    return cap_rows < tk ? cap_rows : tk;
}

size_t esize(const moe_desc& d) { return d.dtype == MOE_BF16 ? 2 : 4; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }


// Route workspace: per-group kept counts, kept lists, and the router weight (plus the
// shared-expert gate column) rewritten in matrix-core fragment order for the router GEMM.
struct RouteLayout {
    size_t kcnt, list, wrt, total;
};
RouteLayout route_layout(const moe_desc& d) {
    const int64_t n_sub = d.sub_seq > 0 ? d.T / d.sub_seq : 0;
    RouteLayout l;
    l.kcnt = 0;
    l.list = align256(sizeof(int32_t) * (size_t)(n_sub * d.E));
    const size_t list_bytes = align256(sizeof(int32_t) * 2 * (size_t)(n_sub * d.E) * d.sub_seq);
    l.wrt = l.list + list_bytes;
    const int nb = (d.E + 1 + 15) / 16;
    l.total = l.wrt + align256((size_t)nb * 16 * d.d * 2);
    return l;
}

size_t ws_size(const moe_desc& d, int which) {
    switch (which) {
        case MOE_WS_ROUTE: return route_layout(d).total;
        case MOE_WS_FFN_FWD: return 0;
        case MOE_WS_FFN_BWD: return 2 * align256((size_t)max_rows(d) * d.f * esize(d));
        case MOE_WS_ROUTE_BWD: {
            const int chunk = moe::router_bwd_chunk(d.dtype);
            const int64_t chunks = (d.T + chunk - 1) / chunk;
            const int64_t ncol8 = (d.E + 1 + 7) / 8 * 8;
            return align256((size_t)chunks * d.d * ncol8 * sizeof(float));
        }
        case MOE_WS_PERMUTE_BWD:  // a transposed router weight, unless it is staged in LDS
            return d.E + 1 <= moe::kPermuteBwdSliceCols ? 0
                                                        : align256((size_t)(d.E + 1) * d.d * esize(d));
        default: return (size_t)-1;
    }
}

moe_status check_ws(const moe_desc& d, int which, const void* ws, size_t bytes) {
    const size_t need = ws_size(d, which);
    REQUIRE(bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", bytes, need);
    REQUIRE(need == 0 || ws, MOE_ERR_INVALID_ARG, "workspace is NULL");
    return MOE_OK;
}

__global__ void zero_counts_kernel(int32_t* kept_counts, int32_t* offsets, int32_t* n_kept,
                                   int E) {
    int i = threadIdx.x;
    if (i < E) kept_counts[i] = 0;
    if (i <= E) offsets[i] = 0;
    if (i == 0) n_kept[0] = 0;
}

bool use_mfma(const moe_desc& d) {
    return !(d.flags & MOE_FLAG_VALU_GEMM) && moe::mfma_shape_ok(d);
}

hipError_t run_gemm(const moe_desc& d, moe::GemmMode mode, const moe::GemmArgs& a,
                    hipStream_t s) {
    if (use_mfma(d)) return moe::launch_gemm_mfma(mode, a, s);
    return moe::launch_gemm_valu(mode, d.dtype == MOE_BF16, a, s);
}

moe::GemmArgs gemm_args(const moe_desc& d, const int32_t* offsets) {
    moe::GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.E = d.E;
    a.R = (int)max_rows(d);
    a.d = d.d;
    a.f = d.f;
    a.offsets = offsets;
    return a;
}

// Argument checks shared by moe_route and moe_route_noalloc (no HIP call).
moe_status check_route_args(const moe_desc* desc, const void* x, const void* w_router,
                            const void* w_sg, const float* logits_out,
                            const float* sg_logit_out, const moe_routing* r) {
    moe_status st;
    if ((st = check_desc(desc)) != MOE_OK) return st;
    if ((st = check_routing(r, desc->T)) != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    REQUIRE(x && w_router && logits_out, MOE_ERR_INVALID_ARG, "x, w_router or logits_out is NULL");
    REQUIRE(!w_sg || sg_logit_out, MOE_ERR_INVALID_ARG, "w_sg given without sg_logit_out");
    return MOE_OK;
}

// The router, softmax/top-K, drop and maps launches of a validated call; `w` is the
// route workspace (route_layout), unused when T == 0.
moe_status route_launch(const moe_desc& d, const void* x, const void* w_router, const float* bias,
                        const void* w_sg, float* logits_out, float* sg_logit_out,
                        const moe_routing& r, char* w, hipStream_t s) {
    if (d.T == 0) {
        zero_counts_kernel<<<1, 128, 0, s>>>(r.kept_counts, r.offsets, r.n_kept, d.E);
        return hip_status(hipGetLastError(), "moe_route");
    }
    const RouteLayout l = route_layout(d);
    hipError_t e = moe::launch_router_fwd(d, x, w_router, bias, w_sg, logits_out, sg_logit_out,
                                          r, s, w + l.wrt);
    if (e != hipSuccess) return hip_status(e, "router");
    moe::RouteWs rw{(int32_t*)(w + l.kcnt), (int32_t*)(w + l.list)};
    return hip_status(moe::launch_select_and_maps(d, r, rw, s), "select/maps");
}

// Route scratch of moe_route_noalloc: one copy per GPU, held until the process ends.
// Every call on a GPU reuses that GPU's copy (calls that overlap on one GPU race).
// Nothing in it has to start at zero: the select kernels write every per-group count
// and the kept lists before the maps kernel reads them, and the router weight in
// matrix-core fragment order is rewritten by each call.
static __device__ __align__(256) char scratch[MOE_ROUTE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices];  // device address of `scratch` on each GPU

// Device address of the current GPU's `scratch` (looked up once per GPU).  The host-side
// name `scratch` is only a handle for the lookup, never an address to pass to a kernel.
moe_status scratch_ptr(char** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED, "device %d >= %d", dev,
            kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        g_scratch_dev[dev] = (char*)p;
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err.c_str(); }

int32_t moe_capacity(int32_t S, int32_t K, int32_t E, double cf) {
    if (cf < 0.0) return -1;
    if (S < 0 || K < 1 || E < 1) return -1;
    return (int32_t)ceil(cf * (double)S * (double)K / (double)E);
}

int64_t moe_max_rows(const moe_desc* desc) {
    if (check_desc(desc) != MOE_OK) return -1;
    return max_rows(*desc);
}

size_t moe_workspace_size(const moe_desc* desc, int32_t which) {
    if (check_desc(desc) != MOE_OK) return (size_t)-1;
    return ws_size(*desc, which);
}

moe_status moe_route(const moe_desc* desc, const void* x, const void* w_router,
                     const float* bias, const void* w_sg, float* logits_out,
                     float* sg_logit_out, const moe_routing* r, void* ws, size_t ws_bytes,
                     void* stream) {
    moe_status st;
    if ((st = check_route_args(desc, x, w_router, w_sg, logits_out, sg_logit_out, r)) != MOE_OK)
        return st;
    if (desc->T > 0 && (st = check_ws(*desc, MOE_WS_ROUTE, ws, ws_bytes)) != MOE_OK) return st;
    return route_launch(*desc, x, w_router, bias, w_sg, logits_out, sg_logit_out, *r, (char*)ws,
                        (hipStream_t)stream);
}

moe_status moe_route_noalloc(const moe_desc* desc, const void* x, const void* w_router,
                             const float* bias, const void* w_sg, float* logits_out,
                             float* sg_logit_out, const moe_routing* r, void* stream) {
    moe_status st;
    if ((st = check_route_args(desc, x, w_router, w_sg, logits_out, sg_logit_out, r)) != MOE_OK)
        return st;
    const size_t need = desc->T > 0 ? ws_size(*desc, MOE_WS_ROUTE) : 0;
    REQUIRE(need <= MOE_ROUTE_SCRATCH_BYTES, MOE_ERR_UNSUPPORTED,
            "moe_route_noalloc: this shape needs %zu bytes of route scratch, more than the "
            "library's fixed %zu (use moe_route with a workspace)",
            need, (size_t)MOE_ROUTE_SCRATCH_BYTES);
    char* w = nullptr;
    if (need > 0 && (st = scratch_ptr(&w)) != MOE_OK) return st;
    return route_launch(*desc, x, w_router, bias, w_sg, logits_out, sg_logit_out, *r, w,
                        (hipStream_t)stream);
}

moe_status moe_route_from_logits(const moe_desc* desc, const float* logits, const moe_routing* r,
                                 void* ws, size_t ws_bytes, void* stream) {
    moe_status st;
    if ((st = check_desc(desc)) != MOE_OK) return st;
    if ((st = check_routing(r, desc->T)) != MOE_OK) return st;
    const moe_desc& d = *desc;
    hipStream_t s = (hipStream_t)stream;
    if (d.T == 0) {
        zero_counts_kernel<<<1, 128, 0, s>>>(r->kept_counts, r->offsets, r->n_kept, d.E);
        return hip_status(hipGetLastError(), "moe_route_from_logits");
    }
    REQUIRE(logits, MOE_ERR_INVALID_ARG, "logits is NULL");
    if ((st = check_ws(d, MOE_WS_ROUTE, ws, ws_bytes)) != MOE_OK) return st;
    const RouteLayout l = route_layout(d);
    char* w = (char*)ws;
    hipError_t e = moe::launch_topk_from_logits(d, logits, *r, s);
    if (e != hipSuccess) return hip_status(e, "topk");
    moe::RouteWs rw{(int32_t*)(w + l.kcnt), (int32_t*)(w + l.list)};
    return hip_status(moe::launch_select_and_maps(d, *r, rw, s), "select/maps");
}

moe_status moe_permute(const moe_desc* desc, const void* x, const moe_routing* r, void* xp_out,
                       void* stream) {
    moe_status st;
    if ((st = check_desc(desc)) != MOE_OK) return st;
    if ((st = check_routing(r, desc->T)) != MOE_OK) return st;
    if (max_rows(*desc) == 0) return MOE_OK;
    REQUIRE(x && xp_out, MOE_ERR_INVALID_ARG, "x or xp_out is NULL");
    return hip_status(
        moe::launch_permute(*desc, max_rows(*desc), x, *r, xp_out, (hipStream_t)stream),
        "moe_permute");
}

moe_status moe_expert_ffn_fwd(const moe_desc* desc, const void* xp, const void* w_gate,
                              const void* w_up, const void* w_down, const int32_t* offsets,
                              void* a_out, void* b_out, void* h_out, void* o_out, void* ws,
                              size_t ws_bytes, void* stream) {
    moe_status st;
    if ((st = check_desc(desc)) != MOE_OK) return st;
    const moe_desc& d = *desc;
    if (max_rows(d) == 0) return MOE_OK;
    REQUIRE(xp && w_gate && w_up && w_down && offsets && a_out && b_out && h_out && o_out,
            MOE_ERR_INVALID_ARG, "a pointer argument of moe_expert_ffn_fwd is NULL");
    if ((st = check_ws(d, MOE_WS_FFN_FWD, ws, ws_bytes)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    moe::GemmArgs a = gemm_args(d, offsets);
    a.A0 = xp; a.B0 = w_gate; a.B1 = w_up; a.C0 = a_out; a.C1 = b_out; a.C2 = h_out;
    hipError_t e = run_gemm(d, moe::GG_FWD_GATEUP, a, s);
    if (e != hipSuccess) return hip_status(e, "gate/up GEMM");
    moe::GemmArgs b = gemm_args(d, offsets);
    b.A0 = h_out; b.B0 = w_down; b.C0 = o_out;
    b.out_f32 = (d.flags & MOE_FLAG_F32_PARTIAL) != 0;
    return hip_status(run_gemm(d, moe::GG_FWD_DOWN, b, s), "down GEMM");
}

moe_status moe_unpermute(const moe_desc* desc, const void* o, const moe_routing* r,
                         const void* shared_out, const float* sg_logit, void* y_out,
                         void* stream) {
    moe_status st;
    if ((st = check_desc(desc)) != MOE_OK) return st;
    if ((st = check_no_partial(*desc, "moe_unpermute")) != MOE_OK) return st;
    if ((st = check_routing(r, desc->T)) != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    REQUIRE((o || max_rows(*desc) == 0) && y_out, MOE_ERR_INVALID_ARG, "o or y_out is NULL");
    REQUIRE(!shared_out || sg_logit, MOE_ERR_INVALID_ARG, "shared_out given without sg_logit");
    return hip_status(moe::launch_unpermute(*desc, o, *r, shared_out, sg_logit, y_out,
                                            (hipStream_t)stream),
                      "moe_unpermute");
}

moe_status moe_unpermute_bwd(const moe_desc* desc, const void* dy, const void* o,
                             const moe_routing* r, const void* shared_out, const float* sg_logit,
                             void* d_o_out, float* dgate_out, void* dshared_out,
                             float* dsg_logit_out, void* stream) {
    moe_status st;
    if ((st = check_desc(desc)) != MOE_OK) return st;
    if ((st = check_no_partial(*desc, "moe_unpermute_bwd")) != MOE_OK) return st;
    if ((st = check_routing(r, desc->T)) != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    REQUIRE(dy && dgate_out && ((o && d_o_out) || max_rows(*desc) == 0), MOE_ERR_INVALID_ARG,
            "dy, o, d_o_out or dgate_out is NULL");
    REQUIRE(!shared_out || (sg_logit && dshared_out && dsg_logit_out), MOE_ERR_INVALID_ARG,
            "shared_out needs sg_logit, dshared_out and dsg_logit_out");
    return hip_status(moe::launch_unpermute_bwd(*desc, dy, o, *r, shared_out, sg_logit, d_o_out,
                                                dgate_out, dshared_out, dsg_logit_out,
                                                (hipStream_t)stream),
                      "moe_unpermute_bwd");
}

moe_status moe_expert_ffn_bwd(const moe_desc* desc, const void* xp, const void* a, const void* b,
                              const void* h, const void* w_gate, const void* w_up,
                              const void* w_down, const int32_t* offsets, const void* d_o,
                              void* dxp_out, void* dw_gate_out, void* dw_up_out,
                              void* dw_down_out, void* ws, size_t ws_bytes, void* stream) {
    moe_status st;
    if ((st = check_desc(desc)) != MOE_OK) return st;
    const moe_desc& d = *desc;
    const bool rows = max_rows(d) > 0;  // without rows only the (zero) weight grads are written
    REQUIRE(offsets && dw_gate_out && dw_up_out && dw_down_out &&
                (!rows || (xp && a && b && h && w_gate && w_up && w_down && d_o && dxp_out)),
            MOE_ERR_INVALID_ARG, "a pointer argument of moe_expert_ffn_bwd is NULL");
    if ((st = check_ws(d, MOE_WS_FFN_BWD, ws, ws_bytes)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const size_t half = ws_size(d, MOE_WS_FFN_BWD) / 2;
    void* da = ws;
    void* db = (char*)ws + half;
    hipError_t e;
    moe::GemmArgs g1 = gemm_args(d, offsets);
    g1.A0 = d_o; g1.B0 = w_down; g1.X0 = a; g1.X1 = b; g1.C0 = da; g1.C1 = db;
    if (rows && (e = run_gemm(d, moe::GG_DGRAD_DOWN, g1, s)) != hipSuccess)
        return hip_status(e, "down dgrad GEMM");
    // The weight gradients are written for every expert, also with no rows (zeros).
    moe::GemmArgs g2 = gemm_args(d, offsets);
    g2.A0 = h; g2.B0 = d_o; g2.C0 = dw_down_out;
    if ((e = run_gemm(d, moe::GG_WGRAD_DOWN, g2, s)) != hipSuccess)
        return hip_status(e, "down wgrad GEMM");
    moe::GemmArgs g3 = gemm_args(d, offsets);
    g3.A0 = xp; g3.B0 = da; g3.B1 = db; g3.C0 = dw_gate_out; g3.C1 = dw_up_out;
    if ((e = run_gemm(d, moe::GG_WGRAD_GATEUP, g3, s)) != hipSuccess)
        return hip_status(e, "gate/up wgrad GEMM");
    moe::GemmArgs g4 = gemm_args(d, offsets);
    g4.A0 = da; g4.A1 = db; g4.B0 = w_gate; g4.B1 = w_up; g4.C0 = dxp_out;
    g4.out_f32 = (d.flags & MOE_FLAG_F32_PARTIAL) != 0;
    if (rows && (e = run_gemm(d, moe::GG_DGRAD_GATEUP, g4, s)) != hipSuccess)
        return hip_status(e, "gate/up dgrad GEMM");
    return MOE_OK;
}

moe_status moe_route_bwd(const moe_desc* desc, const void* x, const moe_routing* r,
                         const float* dgate, const float* dsg_logit, float* dlogits_out,
                         void* dw_router_out, void* dw_sg_out, void* ws, size_t ws_bytes,
                         void* stream) {
    moe_status st;
    if ((st = check_desc(desc)) != MOE_OK) return st;
    if ((st = check_routing(r, desc->T)) != MOE_OK) return st;
    const moe_desc& d = *desc;
    REQUIRE(dw_router_out && (d.T == 0 || (x && dgate && dlogits_out)), MOE_ERR_INVALID_ARG,
            "x, dgate, dlogits_out or dw_router_out is NULL");
    REQUIRE(!dsg_logit || dw_sg_out, MOE_ERR_INVALID_ARG, "dsg_logit given without dw_sg_out");
    if ((st = check_ws(d, MOE_WS_ROUTE_BWD, ws, ws_bytes)) != MOE_OK) return st;
    const int chunk = moe::router_bwd_chunk(d.dtype);
    const int chunks = (d.T + chunk - 1) / chunk;
    return hip_status(moe::launch_router_bwd(d, x, *r, dgate, dsg_logit, dlogits_out,
                                             dw_router_out, dw_sg_out, (float*)ws, chunks,
                                             chunk, (hipStream_t)stream),
                      "moe_route_bwd");
}

moe_status moe_permute_bwd(const moe_desc* desc, const void* dxp, const moe_routing* r,
                           const float* dlogits, const void* w_router, const float* dsg_logit,
                           const void* w_sg, const void* dx_add, void* dx_out, void* ws,
                           size_t ws_bytes, void* stream) {
    moe_status st;
    if ((st = check_desc(desc)) != MOE_OK) return st;
    if ((st = check_no_partial(*desc, "moe_permute_bwd")) != MOE_OK) return st;
    if ((st = check_routing(r, desc->T)) != MOE_OK) return st;
    const moe_desc& d = *desc;
    if (d.T == 0) return MOE_OK;
    REQUIRE((dxp || max_rows(d) == 0) && dx_out, MOE_ERR_INVALID_ARG, "dxp or dx_out is NULL");
    REQUIRE(!dlogits || w_router, MOE_ERR_INVALID_ARG, "dlogits given without w_router");
    REQUIRE(!dsg_logit || w_sg, MOE_ERR_INVALID_ARG, "dsg_logit given without w_sg");
    if ((st = check_ws(d, MOE_WS_PERMUTE_BWD, ws, ws_bytes)) != MOE_OK) return st;
    return hip_status(moe::launch_permute_bwd(d, dxp, *r, dlogits, w_router, dsg_logit, w_sg,
                                              dx_add, dx_out, ws, (hipStream_t)stream),
                      "moe_permute_bwd");
}

}  // extern "C"
