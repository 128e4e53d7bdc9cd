// gdr_launch.hpp -- host-side launchers of the gfx950 kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

// Chunk table: one entry per chunk, chunk-major over sequences.
struct ChunkInfo {
    int seq;  // sequence index
    int t0;   // global token index of the chunk's first row
    int len;  // rows in this chunk (1..BT)
    int pad;  // chunk index within its sequence
};

// Arguments shared by the launchers.  All pointers are device pointers.
struct Problem {
    int B, T, HK, HV, K, V, BT, N;
    int64_t NT;        // total chunks
    float scale;
    int dtype;         // gdr_dtype
    const int32_t* cu; // device cu_seqlens or NULL
};

// Workspace carve-up (byte offsets from the workspace base).
struct WsPlan {
    size_t chunk_info, seq_chunk0, W, U, R, A, KT, h, dh, total;
};
WsPlan plan_workspace(const Problem& p);

hipError_t launch_chunk_table(const Problem& p, ChunkInfo* info, int32_t* seq_chunk0, hipStream_t s);

// K1a: per-chunk WY factors.  W, U, K̃ (and R when q != NULL) in the scan
// operand type; A = (I+L)^{-1} in the input type when A != NULL.
hipError_t launch_prep(const Problem& p, const void* q, const void* k, const void* v, const float* gcum,
                       const void* beta, const ChunkInfo* info, void* W, void* U, void* R, void* A, void* KT,
                       hipStream_t s);

// K1b + K2: the forward state scan and the reverse dh scan (one launch, two roles).
//   fwd role: writes h (state entering each chunk; transposed [NT,HV,V,K] in the
//   input type when hT != NULL, row-major fp32 [NT,HV,K,V] when h32 != NULL),
//   optional v_new (input type) and ht (fp32).
//   rev role (when R != NULL): writes dh (transposed, input type) and dh0.
struct ScanArgs {
    const void* k; const void* dO; const float* gcum; const ChunkInfo* info; const int32_t* seq_chunk0;
    const void* W; const void* U; const void* R; const void* KT;
    const float* h0; const float* dht;
    void* hT; float* h32; void* v_new; float* ht;
    void* dhT; float* dh0;
    const int32_t* cu; int T;   // sequence bounds: cu_seqlens (device) or dense length T
    bool do_fwd, do_rev;
};
hipError_t launch_scans(const Problem& p, const ScanArgs& a, hipStream_t s);

// K3 (+ the tail): per-chunk gradients.
struct GradArgs {
    const void* q; const void* k; const void* v; const float* gcum; const void* beta; const void* dO;
    const void* hT; const void* dhT; const void* A; const ChunkInfo* info;
    void* dq; void* dk; void* dv; float* dg; float* dbeta;
};
hipError_t launch_grad(const Problem& p, const GradArgs& a, hipStream_t s);

// KDA WY backward stage.
struct KdaArgs {
    const void* q; const void* k; const void* v; const void* v_new; const float* g; const void* beta;
    const void* A; const float* h; const void* dO; const float* dh; const void* dv_in;
    const ChunkInfo* info;
    float* dq; float* dk; void* dv_out; float* db; float* dg; float* dA;
};
hipError_t launch_kda(const Problem& p, const KdaArgs& a, hipStream_t s);

}  // namespace gdr
