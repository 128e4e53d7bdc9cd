// bigdn_launch.hpp -- host-side launchers of the BiGDN kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bigdn {

// Sizes: B batch, F frames of S tokens (N = F*S tokens per batch row), H heads
// of dimension D (C = H*D channels).
struct Dims {
    int B, F, S, H, D;
    float k_scale, norm_eps, eps;
};

// Device pointers into the caller's workspace (see plan()).
struct Ws {
    float *rq, *rk;      // [B*N] inverse RMS of q and k over all C channels
    void* P;             // bf16 [NF][D][D]  P_f = Kr^T diag(beta) Kr
    float *A, *Pz, *Bz;  // [NF][D][D], [NF][D][D], [NF][D]
    void *Mf, *Mr;       // bf16 [NF][D][D]  forward (inclusive) / reverse (exclusive) states
    float *zf, *zr;      // [NF][D]
    float *dMc, *dzc;    // [NF][D][D], [NF][D]  gradients of the combined state / normaliser
    void *Tf, *Tr;       // bf16 [NF][D][D]  state gradients of the two scans
    float *tzf, *tzr;    // [NF][D]
    float* wpart;        // [NBLK][2C]  per-block norm-weight gradient partials
    int nblk;
};

// Workspace layout; returns the total byte count.  With base == nullptr only
// the size is computed.  `bwd` false plans the forward's prefix only.
size_t plan(const Dims& d, bool bwd, char* base, Ws* w);

struct Inputs {
    const void* qkv;  // bf16 [B, N, 3, H, D]
    const float *beta, *decay, *qw, *kw, *cos, *sin;
    const void* dout;  // bf16 [B, N, H, D] (backward only)
};
struct Outputs {
    void* out;                 // bf16 [B, N, H, D] (forward)
    void* dqkv;                // bf16 [B, N, 3, H, D] (backward)
    float *dbeta, *ddecay, *dqw, *dkw;
};

// ev: NULL or events recorded on `s` (forward: 5, backward: 8; see bigdn.h).
hipError_t launch_bigdn_fwd(const Dims& d, const Inputs& in, const Outputs& out, const Ws& w, hipStream_t s,
                            hipEvent_t* ev);
hipError_t launch_bigdn_bwd(const Dims& d, const Inputs& in, const Outputs& out, const Ws& w, hipStream_t s,
                            hipEvent_t* ev);

}  // namespace bigdn
