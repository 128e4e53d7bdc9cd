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

// Scan segment table: the chunks of a sequence are cut into segments of L
// chunks (the last one shorter) so that the sequential state scans can run
// one workgroup per segment (see gdr_scan.hip).
struct SegInfo {
    int seq;  // sequence index
    int c0;   // global index of the segment's first chunk
    int nc;   // chunks in the segment
    int lc0;  // index of its first chunk within the sequence
};

// Arguments shared by the launchers.  All pointers are device pointers.
struct Problem {
    int B, T, HK, HV, K, V, BT, N;
    int64_t NT;        // total chunks
    float scale;
    int dtype;         // gdr_dtype
    const int32_t* cu; // device cu_seqlens or NULL
    int L;             // scan segment length in chunks
    int NS;            // total scan segments
    int maxS;          // most segments in one sequence (1: no segmented scans)
    int64_t maxC;      // most chunks in one sequence
};

// Workspace carve-up (byte offsets from the workspace base).  The segment
// state buffers (hloc, dhloc, P, hstart, dhin: [NS][HV][K][V] fp32 each, in
// the fp32 fragment order below; P holds its values in the 16-bit operand
// type, in the first half of each block, and its transpose in the second) are
// empty when maxS == 1.
struct WsPlan {
    size_t chunk_info, seq_chunk0, seg_info, seq_seg0, seg_order, W, U, R, A, KT, h, dh;
    size_t hloc, dhloc, P, hstart, dhin, cmax, hmax, dsc, total;
};
WsPlan plan_workspace(const Problem& p);

// seg_order (NULL: not wanted): the segments ranked by descending chunk count,
// ties by index, when there are at most 1024 of them (index order otherwise).
hipError_t launch_chunk_table(const Problem& p, ChunkInfo* info, int32_t* seq_chunk0, SegInfo* seg,
                              int32_t* seq_seg0, int32_t* seg_order, hipStream_t s);

// K1a: per-chunk WY factors.  W, U, K̃ (and R when q != NULL) in the scan
// operand type; A = (I+L)^{-1} in the input type when A != NULL.
hipError_t launch_prep(const Problem& p, const void* q, const void* k, const void* v, const float* gcum,
                       const void* beta, const ChunkInfo* info, void* W, void* U, void* R, void* A, void* KT,
                       hipStream_t s);

// Workspace layout of the per-chunk states h[c] / dh[c] (one K x V block per
// (chunk, value head) unit), shared by the scans (writers) and the gradient
// kernel (reader):
//   16-bit types: the scan's accumulator fragment order.  Element (key k,
//     column v) sits at
//         ((v/16 * K/32 + k/32) * 64 + 16 g + v%16) * 8 + i,
//     with j = k % 32, g = (j % 16) / 4 and i = j % 4 + (j >= 16 ? 4 : 0);
//     so one wave writes each [16 columns x 32 keys] block as 64 lanes x 16 B.
//   fp32: transposed [V][K].
__host__ __device__ constexpr long state_frag_offset(int KD, int k, int v) {
    return ((long)((v / 16) * (KD / 32) + k / 32) * 64 + 16 * ((k % 16) / 4) + v % 16) * 8 + k % 4 +
           ((k % 32) >= 16 ? 4 : 0);
}

// fp32 fragment order of a K x V block (segment buffers): 16 x 16 tiles,
// tile (column block v/16, row block k/16) at ((v/16) * K/16 + k/16) * 256,
// inside it lane 16 g + v%16 holds rows 4g .. 4g+3 (k % 16 = 4 g + e) as 4
// consecutive floats.
__host__ __device__ constexpr long state32_frag_offset(int KD, int k, int v) {
    return ((long)((v / 16) * (KD / 16) + k / 16) * 64 + 16 * ((k % 16) / 4) + v % 16) * 4 + k % 4;
}

// K1b + K2: the forward state scan and the reverse dh scan.
//   fwd role: writes h (state entering each chunk, layout above, in the input
//   type when hT != NULL; row-major fp32 [NT,HV,K,V] when h32 != NULL),
//   optional v_new (input type) and ht (fp32).
//   rev role: writes dh (layout above, input type) and dh0.
// With maxS > 1 three launches: local segment scans and transfer matrices,
// the sequential combine over segments, then the scans proper from the exact
// segment boundary states.
struct ScanArgs {
    const void* dO; const float* gcum; const int32_t* seq_chunk0;
    const SegInfo* seg; const int32_t* seq_seg0;
    const int32_t* seg_order;   // segments by descending chunk count (ties by index), or NULL: index order
    const void* W; const void* U; const void* R; const void* KT;
    const float* h0; const float* dht;
    void* hT; float* h32; void* v_new; float* ht;
    void* dhT; float* dh0;
    float* hloc; float* dhloc; float* P; float* hstart; float* dhin;   // segment buffers
    const int32_t* cu; int T;   // sequence bounds: cu_seqlens (device) or dense length T
    bool do_fwd, do_rev;
    // reverse scans with 16-bit operands: dO and the state are scaled per
    // (sequence, value head) by a power of two so that max(|dO|, |dht|)
    // lands in [1/2, 1) before the fp16 narrowing (NULL: no scaling); the
    // per-chunk states dh[c] are written in that scaled form, dh0 unscaled.
    // cmax [NT][4][HV] and hmax [N][HV] are the per-quarter-chunk / per-sequence
    // maxima of |dO| and |dht|, dsc [N][HV] the scales; info is the chunk table.
    const ChunkInfo* info; float* cmax; float* hmax; float* dsc;
};
hipError_t launch_scans(const Problem& p, const ScanArgs& a, hipStream_t s);
// dmax + dscale: the power-of-two scales the reverse scans of a 16-bit
// problem run dO and dht under (a.dsc); launch before launch_scans
hipError_t launch_scan_scales(const Problem& p, const ScanArgs& a, hipStream_t s);

// K3 (+ the tail): per-chunk gradients.
struct GradArgs {
    const void* q; const void* k; const void* v; const float* gcum; const void* beta; const void* dO;
    const void* hT; const void* dhT; const void* A; const ChunkInfo* info;
    void* dq; void* dk; void* dv; float* dg; float* dbeta;
    const float* dsc;   // [N][HV] scale of dhT (dh[c] stored times it), or NULL (1)
};
hipError_t launch_grad(const Problem& p, const GradArgs& a, hipStream_t s);

// Chunked forward output: o = scale·diag(γ)Q h[c] + scale·lower(Γ⊙QKᵀ)(U − W h[c])
// per (chunk, value head), from the WY factors W, U (scan operand type) and the
// states h[c] written by the forward scan (workspace layout above).
struct FwdArgs {
    const void* q; const void* k; const float* gcum; const ChunkInfo* info;
    const void* W; const void* U; const void* hT; void* o;
};
hipError_t launch_fwd_out(const Problem& p, const FwdArgs& a, hipStream_t s);

// In-chunk cumulative sum of the raw gate (fp32, token order).
hipError_t launch_gate_cumsum(const Problem& p, const float* g, float* gc, hipStream_t s);

// KDA WY backward stage.
struct KdaArgs {
    const void* q; const void* k; const void* v; const void* v_new; const float* g; const void* beta;
    const void* A; const float* h; const void* dO; const float* dh; const void* dv_in;
    const ChunkInfo* info;
    float* dq; float* dk; void* dv_out; float* db; float* dg; float* dA;
};
hipError_t launch_kda(const Problem& p, const KdaArgs& a, hipStream_t s);

// Full KDA backward (kda_full.hip): arguments of all its launches.  Device
// pointers; workspace arrays: W, K̃, Qg [NT*H][64][K] and U [NT*H][64][V] and
// Aqk [NT*H][64][64] in the operand type; A [B*T,H,64], V_new and dV_new
// [B*T,H,V] in the input type; h[c], dh[c] [NT,H,K,V] fp32; the WY stage's
// partials dq, dk, dg [B*T,H,K], dβ [B*T,H], dA [B*T,H,64] fp32.
struct KdaFullArgs {
    const void* q; const void* k; const void* v; const float* gcum; const void* beta; const void* dO;
    const float* h0; const float* dht;
    const ChunkInfo* info; const int32_t* seq_chunk0;
    void* W; void* U; void* KT; void* QG; void* Aqk; void* A;
    float* hs; float* dhs; void* vn; void* dvn;
    float* dqs; float* dks; float* dgs; float* dbs; float* dA;
    void* dq; void* dk; void* dv; float* dg; float* dbeta; float* dh0;
};
// ev: NULL or 5 events; [1..4] are recorded after the WY factors, the scans,
// the WY stage and the intra-chunk kernel ([0] is the caller's).
hipError_t launch_kda_full(const Problem& p, const KdaFullArgs& a, hipStream_t s, hipEvent_t* ev);

}  // namespace gdr
