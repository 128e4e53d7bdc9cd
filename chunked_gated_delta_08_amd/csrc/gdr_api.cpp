// gdr_api.cpp -- the C ABI (include/gdr.h): host-side validation, workspace
// plan and the launch sequence.  Nothing here allocates device memory.
#include <math.h>
#include <string.h>

#include "../../include/gdr.h"
#include "gdr_launch.hpp"

namespace {

using gdr::Problem;
using gdr::SegInfo;
using gdr::WsPlan;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Segments for the sequential state scans.  A sequence of n chunks is cut into
// ceil(n / L) segments (at least one).  Without segments the scans take one
// workgroup per (sequence, value head, direction) and as many sequential
// steps as the longest sequence has chunks; with segments there are three
// launches (local scans and transfer matrices: 2 workgroups per segment and
// value head of every sequence that has more than one segment; the sequential
// combine: one step per segment; the scans proper: 2 workgroups per segment
// and value head).  `dirs` is 2 for the backward and 1 for the forward calls,
// which scan in one direction only (half the workgroups of each launch).  L is chosen to minimise the estimated time in units of one
// chunk step of a round of workgroups (one workgroup per CU on 256 CUs); a
// combine step counts 1.4 such units.  That weight, and counting the local
// scans by workgroups, fit the measured call times at T = 32768 with 16 and 32
// value heads and at the 12-sequence varlen workload (K = V = 128, bf16) over
// L = 8 .. 128.
void plan_segments(const gdr_problem* p, Problem* q, int dirs) {
    const int nseq = q->N;
    auto nch = [&](int n) -> int64_t {
        const int64_t len = p->cu_seqlens ? (int64_t)p->cu_seqlens_host[n + 1] - p->cu_seqlens_host[n] : p->T;
        return (len + p->BT - 1) / p->BT;
    };
    int64_t maxn = 0;
    for (int n = 0; n < nseq; n++) maxn = nch(n) > maxn ? nch(n) : maxn;
    auto rounds = [](int64_t jobs) { return (double)((jobs + 255) / 256); };
    struct Plan { int L; int64_t NS; int maxS; double cost; };
    auto eval = [&](int64_t L) {
        Plan pl{(int)L, 0, 1, 0.0};
        int64_t multi = 0;   // segments of the sequences cut into more than one
        for (int n = 0; n < nseq; n++) {
            const int64_t c = nch(n), S = c > L ? (c + L - 1) / L : 1;
            pl.NS += S;
            if (S > 1) multi += S;
            if (S > pl.maxS) pl.maxS = (int)S;
        }
        const double Ls = (double)(L < maxn ? L : maxn);
        pl.cost = rounds(dirs * q->HV * pl.NS) * Ls;
        if (pl.maxS > 1) pl.cost += rounds(dirs * q->HV * multi) * Ls + 1.4 * pl.maxS;
        return pl;
    };
    Plan best = eval(maxn > 0 ? maxn : 1);   // no segments
    if (q->dtype != GDR_F32 && p->seg_chunks >= 0 && maxn > 1) {
        if (p->seg_chunks > 0) {
            best = eval(p->seg_chunks);
        } else {
            for (int64_t L = 8; L < maxn; L *= 2) {
                const Plan c = eval(L);
                if (c.cost < best.cost) best = c;
            }
        }
    }
    q->L = best.L;
    q->NS = (int)best.NS;
    q->maxS = best.maxS;
}
size_t elem_size(int dtype) { return dtype == GDR_F32 ? 4 : 2; }

// Host-side checks shared by every entry point.  Fills `q` on success.
int check_problem(const gdr_problem* p, Problem* q, int dirs = 2) {
    if (!p) return GDR_ERR_INVALID;
    if (p->B < 1 || p->T < 0 || p->HK < 1 || p->HV < 1 || p->K < 1 || p->V < 1 || p->BT < 1) return GDR_ERR_INVALID;
    if (p->HV % p->HK != 0) return GDR_ERR_INVALID;
    if (p->dtype != GDR_F32 && p->dtype != GDR_F16 && p->dtype != GDR_BF16) return GDR_ERR_INVALID;
    int64_t nt = 0, maxc = 0;
    int nseq;
    if (p->cu_seqlens) {
        if (!p->cu_seqlens_host || p->B != 1 || p->N < 1) return GDR_ERR_INVALID;
        const int32_t* cu = p->cu_seqlens_host;
        if (cu[0] != 0) return GDR_ERR_INVALID;
        for (int n = 0; n < p->N; n++) {
            if (cu[n + 1] < cu[n]) return GDR_ERR_INVALID;
            const int64_t c = (cu[n + 1] - cu[n] + p->BT - 1) / p->BT;
            nt += c;
            maxc = c > maxc ? c : maxc;
        }
        if (cu[p->N] != p->T) return GDR_ERR_INVALID;
        nseq = p->N;
    } else {
        maxc = (p->T + p->BT - 1) / p->BT;
        nt = (int64_t)p->B * maxc;
        nseq = p->B;
    }
    if ((int64_t)p->B * p->T > INT32_MAX / 2) return GDR_ERR_UNSUPPORTED;
    q->B = p->B; q->T = p->T; q->HK = p->HK; q->HV = p->HV; q->K = p->K; q->V = p->V; q->BT = p->BT;
    q->N = nseq; q->NT = nt; q->maxC = maxc;
    q->scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->K);
    q->dtype = p->dtype;
    q->cu = p->cu_seqlens;
    plan_segments(p, q, dirs);
    return GDR_OK;
}

int check_supported(const Problem& q) {
    if (q.BT != 64) return GDR_ERR_UNSUPPORTED;
    if (q.K != q.V || (q.K != 64 && q.K != 128)) return GDR_ERR_UNSUPPORTED;
    if (q.dtype == GDR_F32 && q.K != 64) return GDR_ERR_UNSUPPORTED;
    return GDR_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH; }

void set_seg_buffers(gdr::ScanArgs& a, char* base, const WsPlan& w) {
    a.hloc = (float*)(base + w.hloc); a.dhloc = (float*)(base + w.dhloc); a.P = (float*)(base + w.P);
    a.hstart = (float*)(base + w.hstart); a.dhin = (float*)(base + w.dhin);
}

}  // namespace

namespace gdr {

WsPlan plan_workspace(const Problem& p) {
    WsPlan w{};
    const size_t es = elem_size(p.dtype);       // input type and scan operand type share a width
    const size_t units = (size_t)p.NT * p.HV;
    size_t off = 0;
    w.chunk_info = off; off = align256(off + (size_t)(p.NT > 0 ? p.NT : 1) * sizeof(ChunkInfo));
    w.seq_chunk0 = off; off = align256(off + (size_t)(p.N + 1) * 4);
    w.seg_info = off; off = align256(off + (size_t)p.NS * sizeof(SegInfo));
    w.seq_seg0 = off; off = align256(off + (size_t)(p.N + 1) * 4);
    w.seg_order = off; off = align256(off + (size_t)p.NS * 4);
    w.W = off; off = align256(off + units * 64 * p.K * es);
    w.U = off; off = align256(off + units * 64 * p.V * es);
    w.R = off; off = align256(off + units * 64 * p.K * es);
    w.A = off; off = align256(off + units * 64 * 64 * es);
    w.KT = off; off = align256(off + units * 64 * p.K * es);
    w.h = off; off = align256(off + units * (size_t)p.K * p.V * es);
    w.dh = off; off = align256(off + units * (size_t)p.K * p.V * es);
    const size_t segbuf = p.maxS > 1 ? (size_t)p.NS * p.HV * p.K * p.V * 4 : 0;
    w.hloc = off; off = align256(off + segbuf);
    w.dhloc = off; off = align256(off + segbuf);
    w.P = off; off = align256(off + segbuf);
    w.hstart = off; off = align256(off + segbuf);
    w.dhin = off; off = align256(off + segbuf);
    w.cmax = off; off = align256(off + (size_t)(p.NT > 0 ? p.NT : 1) * 4 * p.HV * 4);
    w.hmax = off; off = align256(off + (size_t)p.N * p.HV * 4);
    w.dsc = off; off = align256(off + (size_t)p.N * p.HV * 4);
    w.total = off;
    return w;
}

}  // namespace gdr

namespace {

// Workspace carve-up of the full KDA backward (byte offsets).
struct KdaWsPlan {
    size_t chunk_info, seq_chunk0, seg_info, seq_seg0, W, U, KT, QG, Aqk, A, hs, dhs, vn, dvn, dqs, dks, dgs, dbs,
        dA, total;
};

KdaWsPlan plan_kda_workspace(const Problem& p) {
    KdaWsPlan w{};
    const size_t es = elem_size(p.dtype);
    const size_t units = (size_t)p.NT * p.HV;
    const size_t ntok = p.cu ? (size_t)p.T : (size_t)p.B * p.T;
    const size_t H = p.HV;
    size_t off = 0;
    w.chunk_info = off; off = align256(off + (size_t)(p.NT > 0 ? p.NT : 1) * sizeof(gdr::ChunkInfo));
    w.seq_chunk0 = off; off = align256(off + (size_t)(p.N + 1) * 4);
    w.seg_info = off; off = align256(off + (size_t)p.NS * sizeof(SegInfo));
    w.seq_seg0 = off; off = align256(off + (size_t)(p.N + 1) * 4);
    w.W = off; off = align256(off + units * 64 * p.K * es);
    w.U = off; off = align256(off + units * 64 * p.V * es);
    w.KT = off; off = align256(off + units * 64 * p.K * es);
    w.QG = off; off = align256(off + units * 64 * p.K * es);
    w.Aqk = off; off = align256(off + units * 64 * 64 * es);
    w.A = off; off = align256(off + ntok * H * 64 * es);
    w.hs = off; off = align256(off + units * (size_t)p.K * p.V * 4);
    w.dhs = off; off = align256(off + units * (size_t)p.K * p.V * 4);
    w.vn = off; off = align256(off + ntok * H * p.V * es);
    w.dvn = off; off = align256(off + ntok * H * p.V * es);
    w.dqs = off; off = align256(off + ntok * H * p.K * 4);
    w.dks = off; off = align256(off + ntok * H * p.K * 4);
    w.dgs = off; off = align256(off + ntok * H * p.K * 4);
    w.dbs = off; off = align256(off + ntok * H * 4);
    w.dA = off; off = align256(off + ntok * H * 64 * 4);
    w.total = off;
    return w;
}

// Validation of the full KDA backward: one head count, K = V in {64, 128},
// fp16 (or fp32 at K = 64), BT = 64; the scans are never segmented.
int check_kda_full(const gdr_problem* p, Problem* q) {
    if (!p) return GDR_ERR_INVALID;
    gdr_problem pp = *p;
    pp.seg_chunks = -1;
    int st = check_problem(&pp, q);
    if (st != GDR_OK) return st;
    if (q->HK != q->HV) return GDR_ERR_INVALID;
    if (q->BT != 64 || q->K != q->V || (q->K != 64 && q->K != 128)) return GDR_ERR_UNSUPPORTED;
    if (q->dtype == GDR_BF16 || (q->dtype == GDR_F32 && q->K != 64)) return GDR_ERR_UNSUPPORTED;
    return GDR_OK;
}

}  // namespace

extern "C" {

const char* gdr_strerror(int status) {
    switch (status) {
        case GDR_OK: return "ok";
        case GDR_ERR_INVALID: return "invalid argument (shape, dtype, null pointer or cu_seqlens)";
        case GDR_ERR_UNSUPPORTED: return "unsupported configuration (the library handles BT=64, K=V in {64,128}; fp32 only at K=64)";
        case GDR_ERR_WORKSPACE: return "workspace missing or smaller than gdr_workspace_size()";
        case GDR_ERR_LAUNCH: return "HIP error at kernel launch";
        case GDR_ERR_SCRATCH: return "problem needs more workspace than the fixed scratch of gdr_chunk_bwd_noalloc";
        default: return "unknown status";
    }
}

int64_t gdr_num_chunks(const gdr_problem* p) {
    Problem q;
    if (check_problem(p, &q) != GDR_OK) return -1;
    return q.NT;
}

size_t gdr_workspace_size(const gdr_problem* p) {
    // large enough for the segment plans of both the forward and the backward
    // calls; every GDN entry point asks for at least this much
    Problem q1, q2;
    if (check_problem(p, &q1, 1) != GDR_OK || check_problem(p, &q2, 2) != GDR_OK) return 0;
    const size_t a = gdr::plan_workspace(q1).total, b = gdr::plan_workspace(q2).total;
    return a > b ? a : b;
}

int gdr_fwd_states(const gdr_problem* p, const void* k, const void* v, const float* g_cum, const void* beta,
                   const float* h0, float* h_out, void* v_new_out, float* ht_out, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
    Problem q;
    int st = check_problem(p, &q, 1);
    if (st != GDR_OK) return st;
    if ((st = check_supported(q)) != GDR_OK) return st;
    if (q.NT > 0 && (!k || !v || !g_cum || !beta || !h_out)) return GDR_ERR_INVALID;
    const WsPlan w = gdr::plan_workspace(q);
    if (!ws || ws_bytes < gdr_workspace_size(p)) return GDR_ERR_WORKSPACE;
    char* base = (char*)ws;
    auto* info = (gdr::ChunkInfo*)(base + w.chunk_info);
    auto* sc0 = (int32_t*)(base + w.seq_chunk0);
    auto* seg = (SegInfo*)(base + w.seg_info);
    auto* ss0 = (int32_t*)(base + w.seq_seg0);
    auto* sord = (int32_t*)(base + w.seg_order);
    if ((st = launch_status(gdr::launch_chunk_table(q, info, sc0, seg, ss0, sord, stream))) != GDR_OK) return st;
    if (q.NT > 0) {
        st = launch_status(gdr::launch_prep(q, nullptr, k, v, g_cum, beta, info, base + w.W, base + w.U, nullptr,
                                            nullptr, base + w.KT, stream));
        if (st != GDR_OK) return st;
    }
    gdr::ScanArgs a{};
    a.gcum = g_cum; a.seq_chunk0 = sc0; a.seg = seg; a.seq_seg0 = ss0; a.seg_order = sord;
    set_seg_buffers(a, base, w);
    a.W = base + w.W; a.U = base + w.U; a.KT = base + w.KT; a.h0 = h0;
    a.h32 = h_out; a.v_new = v_new_out; a.ht = ht_out;
    a.cu = q.cu; a.T = q.T;
    a.do_fwd = true; a.do_rev = false;
    return launch_status(gdr::launch_scans(q, a, stream));
}

int gdr_gate_cumsum(const gdr_problem* p, const float* g, float* g_cum, hipStream_t stream) {
    Problem q;
    int st = check_problem(p, &q);
    if (st != GDR_OK) return st;
    const int64_t n = (p->cu_seqlens ? (int64_t)p->T : (int64_t)p->B * p->T) * p->HV;
    if (n == 0) return GDR_OK;
    if (!g || !g_cum) return GDR_ERR_INVALID;
    if ((const char*)g < (const char*)(g_cum + n) && (const char*)g_cum < (const char*)(g + n)) return GDR_ERR_INVALID;
    return launch_status(gdr::launch_gate_cumsum(q, g, g_cum, stream));
}

int gdr_chunk_fwd_events(const gdr_problem* p, const void* qp, const void* k, const void* v, const float* g_cum,
                         const void* beta, const float* h0, void* o, float* ht_out, void* ws, size_t ws_bytes,
                         hipStream_t stream, hipEvent_t* ev) {
    Problem q;
    int st = check_problem(p, &q, 1);
    if (st != GDR_OK) return st;
    if ((st = check_supported(q)) != GDR_OK) return st;
    if (q.NT > 0 && (!qp || !k || !v || !g_cum || !beta || !o)) return GDR_ERR_INVALID;
    const WsPlan w = gdr::plan_workspace(q);
    if (!ws || ws_bytes < gdr_workspace_size(p)) return GDR_ERR_WORKSPACE;
    char* base = (char*)ws;
    auto* info = (gdr::ChunkInfo*)(base + w.chunk_info);
    auto* sc0 = (int32_t*)(base + w.seq_chunk0);
    auto* seg = (SegInfo*)(base + w.seg_info);
    auto* ss0 = (int32_t*)(base + w.seq_seg0);
    auto* sord = (int32_t*)(base + w.seg_order);
    auto mark = [&](int i) { return ev ? launch_status(hipEventRecord(ev[i], stream)) : GDR_OK; };
    if ((st = mark(0)) != GDR_OK) return st;
    if ((st = launch_status(gdr::launch_chunk_table(q, info, sc0, seg, ss0, sord, stream))) != GDR_OK) return st;
    if (q.NT > 0) {
        st = launch_status(gdr::launch_prep(q, nullptr, k, v, g_cum, beta, info, base + w.W, base + w.U, nullptr,
                                            nullptr, base + w.KT, stream));
        if (st != GDR_OK) return st;
    }
    if ((st = mark(1)) != GDR_OK) return st;
    gdr::ScanArgs a{};
    a.gcum = g_cum; a.seq_chunk0 = sc0; a.seg = seg; a.seq_seg0 = ss0; a.seg_order = sord;
    set_seg_buffers(a, base, w);
    a.W = base + w.W; a.U = base + w.U; a.KT = base + w.KT; a.h0 = h0;
    a.hT = base + w.h; a.ht = ht_out;
    a.cu = q.cu; a.T = q.T;
    a.do_fwd = true; a.do_rev = false;
    if ((st = launch_status(gdr::launch_scans(q, a, stream))) != GDR_OK) return st;
    if ((st = mark(2)) != GDR_OK) return st;
    if (q.NT > 0) {
        gdr::FwdArgs f{};
        f.q = qp; f.k = k; f.gcum = g_cum; f.info = info;
        f.W = base + w.W; f.U = base + w.U; f.hT = base + w.h; f.o = o;
        if ((st = launch_status(gdr::launch_fwd_out(q, f, stream))) != GDR_OK) return st;
    }
    return mark(3);
}

int gdr_chunk_fwd(const gdr_problem* p, const void* qp, const void* k, const void* v, const float* g_cum,
                  const void* beta, const float* h0, void* o, float* ht_out, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
    return gdr_chunk_fwd_events(p, qp, k, v, g_cum, beta, h0, o, ht_out, ws, ws_bytes, stream, nullptr);
}

int gdr_chunk_bwd_events(const gdr_problem* p, const void* qp, const void* k, const void* v, const float* g_cum,
                         const void* beta, const float* h0, const void* dO, const float* dht, void* dq, void* dk,
                         void* dv, float* dg, float* dbeta, float* dh0, void* ws, size_t ws_bytes,
                         hipStream_t stream, hipEvent_t* ev) {
    Problem q;
    int st = check_problem(p, &q);
    if (st != GDR_OK) return st;
    if ((st = check_supported(q)) != GDR_OK) return st;
    if (q.NT > 0 && (!qp || !k || !v || !g_cum || !beta || !dO || !dq || !dk || !dv || !dg || !dbeta))
        return GDR_ERR_INVALID;
    const WsPlan w = gdr::plan_workspace(q);
    if (!ws || ws_bytes < gdr_workspace_size(p)) return GDR_ERR_WORKSPACE;
    char* base = (char*)ws;
    auto* info = (gdr::ChunkInfo*)(base + w.chunk_info);
    auto* sc0 = (int32_t*)(base + w.seq_chunk0);
    auto* seg = (SegInfo*)(base + w.seg_info);
    auto* ss0 = (int32_t*)(base + w.seq_seg0);
    auto* sord = (int32_t*)(base + w.seg_order);
    auto mark = [&](int i) { return ev ? launch_status(hipEventRecord(ev[i], stream)) : GDR_OK; };
    gdr::ScanArgs a{};
    a.dO = dO; a.gcum = g_cum; a.seq_chunk0 = sc0; a.seg = seg; a.seq_seg0 = ss0; a.seg_order = sord;
    set_seg_buffers(a, base, w);
    a.W = base + w.W; a.U = base + w.U; a.R = base + w.R; a.KT = base + w.KT;
    a.h0 = h0; a.dht = dht;
    a.hT = base + w.h; a.dhT = base + w.dh; a.dh0 = dh0;
    a.cu = q.cu; a.T = q.T;
    a.do_fwd = q.NT > 0; a.do_rev = true;
    if (q.dtype != GDR_F32) {   // fp16 scan operands: scale dO and the state per (sequence, head)
        a.info = info;
        a.cmax = (float*)(base + w.cmax); a.hmax = (float*)(base + w.hmax); a.dsc = (float*)(base + w.dsc);
    }
    if ((st = mark(0)) != GDR_OK) return st;
    if ((st = launch_status(gdr::launch_chunk_table(q, info, sc0, seg, ss0, sord, stream))) != GDR_OK) return st;
    // the scales first (they read dO and dht only), then the WY factors
    if ((st = launch_status(gdr::launch_scan_scales(q, a, stream))) != GDR_OK) return st;
    if (q.NT > 0) {
        st = launch_status(gdr::launch_prep(q, qp, k, v, g_cum, beta, info, base + w.W, base + w.U, base + w.R,
                                            base + w.A, base + w.KT, stream));
        if (st != GDR_OK) return st;
    }
    if ((st = mark(1)) != GDR_OK) return st;
    if ((st = launch_status(gdr::launch_scans(q, a, stream))) != GDR_OK) return st;
    if ((st = mark(2)) != GDR_OK) return st;
    if (q.NT > 0) {
        gdr::GradArgs g{};
        g.q = qp; g.k = k; g.v = v; g.gcum = g_cum; g.beta = beta; g.dO = dO;
        g.hT = base + w.h; g.dhT = base + w.dh; g.A = base + w.A; g.info = info;
        g.dq = dq; g.dk = dk; g.dv = dv; g.dg = dg; g.dbeta = dbeta;
        g.dsc = a.dsc;
        st = launch_status(gdr::launch_grad(q, g, stream));
        if (st != GDR_OK) return st;
    }
    return mark(3);
}

int gdr_chunk_bwd(const gdr_problem* p, const void* qp, const void* k, const void* v, const float* g_cum,
                  const void* beta, const float* h0, const void* dO, const float* dht, void* dq, void* dk, void* dv,
                  float* dg, float* dbeta, float* dh0, void* ws, size_t ws_bytes, hipStream_t stream) {
    return gdr_chunk_bwd_events(p, qp, k, v, g_cum, beta, h0, dO, dht, dq, dk, dv, dg, dbeta, dh0, ws, ws_bytes,
                                stream, nullptr);
}

size_t kda_workspace_size(const gdr_problem* p) {
    Problem q;
    if (check_kda_full(p, &q) != GDR_OK) return 0;
    return plan_kda_workspace(q).total;
}

int kda_chunk_bwd_full_events(const gdr_problem* p, const void* qp, const void* k, const void* v, const float* g_cum,
                              const void* beta, const float* h0, const void* dO, const float* dht, void* dq, void* dk,
                              void* dv, float* dg, float* dbeta, float* dh0, void* ws, size_t ws_bytes,
                              hipStream_t stream, hipEvent_t* ev) {
    Problem q;
    int st = check_kda_full(p, &q);
    if (st != GDR_OK) return st;
    if (q.NT > 0 && (!qp || !k || !v || !g_cum || !beta || !dO || !dq || !dk || !dv || !dg || !dbeta))
        return GDR_ERR_INVALID;
    const KdaWsPlan w = plan_kda_workspace(q);
    if (!ws || ws_bytes < w.total) return GDR_ERR_WORKSPACE;
    char* base = (char*)ws;
    auto* info = (gdr::ChunkInfo*)(base + w.chunk_info);
    auto* sc0 = (int32_t*)(base + w.seq_chunk0);
    if (ev && (st = launch_status(hipEventRecord(ev[0], stream))) != GDR_OK) return st;
    st = launch_status(gdr::launch_chunk_table(q, info, sc0, (SegInfo*)(base + w.seg_info),
                                               (int32_t*)(base + w.seq_seg0), nullptr, stream));
    if (st != GDR_OK) return st;
    gdr::KdaFullArgs a{};
    a.q = qp; a.k = k; a.v = v; a.gcum = g_cum; a.beta = beta; a.dO = dO; a.h0 = h0; a.dht = dht;
    a.info = info; a.seq_chunk0 = sc0;
    a.W = base + w.W; a.U = base + w.U; a.KT = base + w.KT; a.QG = base + w.QG; a.Aqk = base + w.Aqk;
    a.A = base + w.A; a.hs = (float*)(base + w.hs); a.dhs = (float*)(base + w.dhs);
    a.vn = base + w.vn; a.dvn = base + w.dvn;
    a.dqs = (float*)(base + w.dqs); a.dks = (float*)(base + w.dks); a.dgs = (float*)(base + w.dgs);
    a.dbs = (float*)(base + w.dbs); a.dA = (float*)(base + w.dA);
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
    return launch_status(gdr::launch_kda_full(q, a, stream, ev));
}

int kda_chunk_bwd_full(const gdr_problem* p, const void* qp, const void* k, const void* v, const float* g_cum,
                       const void* beta, const float* h0, const void* dO, const float* dht, void* dq, void* dk,
                       void* dv, float* dg, float* dbeta, float* dh0, void* ws, size_t ws_bytes, hipStream_t stream) {
    return kda_chunk_bwd_full_events(p, qp, k, v, g_cum, beta, h0, dO, dht, dq, dk, dv, dg, dbeta, dh0, ws, ws_bytes,
                                     stream, nullptr);
}

int kda_chunk_bwd(const gdr_problem* p, const void* qp, const void* k, const void* v, const void* v_new,
                  const float* g, const void* beta, const void* A, const float* h, const void* dO, const float* dh,
                  const void* dv_in, float* dq, float* dk, void* dv_out, float* db, float* dg, float* dA,
                  hipStream_t stream) {
    Problem q;
    int st = check_problem(p, &q);
    if (st != GDR_OK) return st;
    if (q.HK != q.HV) return GDR_ERR_INVALID;
    if (q.dtype == GDR_BF16) return GDR_ERR_UNSUPPORTED;
    if ((q.BT != 64 && q.BT != 16) || q.K != q.V || (q.K != 64 && q.K != 128)) return GDR_ERR_UNSUPPORTED;
    if (q.dtype == GDR_F32 && q.K != 64) return GDR_ERR_UNSUPPORTED;   // fp32 tiles exceed the LDS budget at 128
    if (q.NT == 0) return GDR_OK;
    if (!qp || !k || !v || !v_new || !g || !beta || !A || !h || !dO || !dh || !dv_in || !dq || !dk || !dv_out ||
        !db || !dg || !dA)
        return GDR_ERR_INVALID;
    gdr::KdaArgs a{};
    a.q = qp; a.k = k; a.v = v; a.v_new = v_new; a.g = g; a.beta = beta; a.A = A; a.h = h; a.dO = dO; a.dh = dh;
    a.dv_in = dv_in; a.dq = dq; a.dk = dk; a.dv_out = dv_out; a.db = db; a.dg = dg; a.dA = dA;
    return launch_status(gdr::launch_kda(q, a, stream));
}

}  // extern "C"
