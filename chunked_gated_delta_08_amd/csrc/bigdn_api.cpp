// bigdn_api.cpp -- C ABI of the BiGDN layer (include/bigdn.h): host-side
// validation, workspace carve-up and launch sequencing.
#include <math.h>

#include "bigdn.h"
#include "bigdn_launch.hpp"

namespace {

int check(const bigdn_problem* p, bigdn::Dims* d) {
    if (!p) return GDR_ERR_INVALID;
    if (p->B < 1 || p->F < 1 || p->S < 1 || p->H < 1 || p->D < 1) return GDR_ERR_INVALID;
    if (!isfinite(p->k_scale) || !(p->norm_eps >= 0.f) || !(p->eps > 0.f) || !isfinite(p->norm_eps) ||
        !isfinite(p->eps))
        return GDR_ERR_INVALID;
    if (p->D != 64 && p->D != 128) return GDR_ERR_UNSUPPORTED;
    if ((long)p->H * p->D > 4096) return GDR_ERR_UNSUPPORTED;
    // token and frame counts are kept in int (kernel arguments and grids)
    const long long ntok = (long long)p->B * p->F * p->S;
    if (ntok * 3 * p->H * p->D > (1LL << 40) || ntok > (1LL << 30) ||
        (long long)p->B * p->H * p->F > (1LL << 30))
        return GDR_ERR_UNSUPPORTED;
    *d = bigdn::Dims{p->B, p->F, p->S, p->H, p->D, p->k_scale, p->norm_eps, p->eps};
    return GDR_OK;
}

int status(hipError_t e) { return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH; }

}  // namespace

extern "C" {

size_t bigdn_workspace_size(const bigdn_problem* p, int bwd) {
    bigdn::Dims d;
    if (check(p, &d) != GDR_OK) return 0;
    return bigdn::plan(d, bwd != 0, nullptr, nullptr);
}

int bigdn_fwd_events(const bigdn_problem* p, const void* qkv, const float* beta, const float* decay,
                     const float* q_norm_weight, const float* k_norm_weight, const float* rope_cos,
                     const float* rope_sin, void* out, void* ws, size_t ws_bytes, hipStream_t stream,
                     hipEvent_t* events) {
    bigdn::Dims d;
    int st = check(p, &d);
    if (st != GDR_OK) return st;
    if (!qkv || !beta || !decay || !q_norm_weight || !k_norm_weight || !rope_cos || !rope_sin || !out)
        return GDR_ERR_INVALID;
    bigdn::Ws w;
    const size_t need = bigdn::plan(d, false, nullptr, nullptr);
    if (!ws || ws_bytes < need) return GDR_ERR_WORKSPACE;
    bigdn::plan(d, false, (char*)ws, &w);
    bigdn::Inputs in{qkv, beta, decay, q_norm_weight, k_norm_weight, rope_cos, rope_sin, nullptr};
    bigdn::Outputs o{out, nullptr, nullptr, nullptr, nullptr, nullptr};
    return status(bigdn::launch_bigdn_fwd(d, in, o, w, stream, events));
}

int bigdn_fwd(const bigdn_problem* p, const void* qkv, const float* beta, const float* decay,
              const float* q_norm_weight, const float* k_norm_weight, const float* rope_cos, const float* rope_sin,
              void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    return bigdn_fwd_events(p, qkv, beta, decay, q_norm_weight, k_norm_weight, rope_cos, rope_sin, out, ws, ws_bytes,
                            stream, nullptr);
}

int bigdn_bwd_events(const bigdn_problem* p, const void* qkv, const float* beta, const float* decay,
                     const float* q_norm_weight, const float* k_norm_weight, const float* rope_cos,
                     const float* rope_sin, const void* dout, void* dqkv, float* dbeta, float* ddecay,
                     float* dq_norm_weight, float* dk_norm_weight, void* ws, size_t ws_bytes, hipStream_t stream,
                     hipEvent_t* events) {
    bigdn::Dims d;
    int st = check(p, &d);
    if (st != GDR_OK) return st;
    if (!qkv || !beta || !decay || !q_norm_weight || !k_norm_weight || !rope_cos || !rope_sin || !dout || !dqkv ||
        !dbeta || !ddecay || !dq_norm_weight || !dk_norm_weight)
        return GDR_ERR_INVALID;
    bigdn::Ws w;
    const size_t need = bigdn::plan(d, true, nullptr, nullptr);
    if (!ws || ws_bytes < need) return GDR_ERR_WORKSPACE;
    bigdn::plan(d, true, (char*)ws, &w);
    bigdn::Inputs in{qkv, beta, decay, q_norm_weight, k_norm_weight, rope_cos, rope_sin, dout};
    bigdn::Outputs o{nullptr, dqkv, dbeta, ddecay, dq_norm_weight, dk_norm_weight};
    return status(bigdn::launch_bigdn_bwd(d, in, o, w, stream, events));
}

int bigdn_bwd(const bigdn_problem* p, const void* qkv, const float* beta, const float* decay,
              const float* q_norm_weight, const float* k_norm_weight, const float* rope_cos, const float* rope_sin,
              const void* dout, void* dqkv, float* dbeta, float* ddecay, float* dq_norm_weight,
              float* dk_norm_weight, void* ws, size_t ws_bytes, hipStream_t stream) {
    return bigdn_bwd_events(p, qkv, beta, decay, q_norm_weight, k_norm_weight, rope_cos, rope_sin, dout, dqkv, dbeta,
                            ddecay, dq_norm_weight, dk_norm_weight, ws, ws_bytes, stream, nullptr);
}

}  // extern "C"
