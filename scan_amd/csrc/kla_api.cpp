// kla_api.cpp -- C-ABI front end of the KLA forward library (see include/kla.h).
//
// Validates every argument on the host, before any HIP call, then enqueues
// the gfx950 kernels on the caller's stream.  Nothing here allocates device
// memory or synchronises.
#include "kla.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "kla_bwd.h"
#include "kla_internal.h"
#include "kla_residual.h"
#include "kla_short.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, size_t bytes) { return Span{(uintptr_t)p, (uintptr_t)p + bytes}; }

bool overlap(Span a, Span b) {
    if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool dims_ok(const klaDims* d) {
    return d->B >= 0 && d->H >= 0 && d->T >= 0 && d->dk >= 1 && d->dv >= 1;
}

bool kinds_ok(const klaDims* d) {
    return (d->dtype == KLA_F32 || d->dtype == KLA_BF16) && (d->cov == KLA_DIAG || d->cov == KLA_ISO);
}

bool supported(const klaDims* d) {
    if (!kinds_ok(d)) return false;
    return d->cov == KLA_DIAG ? kla::fwd_diag_supported(d->dk, d->dv, d->dtype)
                              : kla::fwd_iso_supported(d->dk, d->dv, d->dtype);
}

// KLA_FWD_DIAG_IMPL=chunk / KLA_FWD_ISO_IMPL=chunk select the single-role
// chunk kernels for every shape (the wave-specialised kernels are used where
// they are built).
bool use_pipe() {
    const char* s = getenv("KLA_FWD_DIAG_IMPL");
    return !(s && s[0] == 'c');
}
bool use_iso_pipe() {
    const char* s = getenv("KLA_FWD_ISO_IMPL");
    return !(s && s[0] == 'c');
}

int env_vtiles() {
    const char* s = getenv("KLA_FWD_VTILES");
    if (!s || !*s) return 0;
    return atoi(s);
}

// KLA_DIAG_CHAIN=scan runs the diagonal precision of the wave-specialised
// kernel as a wavefront-level Mobius scan (bf16 inputs); default: the
// per-lane serial recursion, which measured faster.
bool use_chain_scan() {
    const char* s = getenv("KLA_DIAG_CHAIN");
    return s && s[0] == 's';
}

// KLA_FWD_SHORT=0 keeps short sequences (T <= kShortTMax) on the chunked
// kernels instead of the short-sequence kernel.
bool use_short() {
    const char* s = getenv("KLA_FWD_SHORT");
    return !(s && s[0] == '0');
}

// KLA_FWD_NSEG=n forces n sequence segments on the wave-specialised diagonal
// kernel (1 = no split); by default long sequences with few (b,h) are split.
int env_nseg() {
    const char* s = getenv("KLA_FWD_NSEG");
    if (!s || !*s) return 0;
    return atoi(s);
}

// Value tiles of the wave-specialised diagonal kernel: 64-column tiles, or,
// for few long sequences that take the sequence split either way, whole
// 128-column rows, so that the chain and gate work is done once per (b,h)
// and segment instead of once per tile (measured 11% faster on the
// B1 H16 T32768 d128 forward).
int diag_pipe_vtiles(const klaDims* d) {
    const int nvt = kla::fwd_diag_pipe_vtiles(d->dk, d->dv, d->dtype);
    if (nvt == 2 && kla::fwd_diag_pipe_supported(d->dk, d->dv, 1, d->dtype) &&
        kla::fwd_diag_nseg(d->B, d->H, d->T, d->dk, d->dv, 2) > 1 &&
        kla::fwd_diag_nseg(d->B, d->H, d->T, d->dk, d->dv, 1) > 1)
        return 1;
    return nvt;
}

// Kernel that klaFwd launches for these (supported) dims; n_vtiles receives
// the number of value-column tiles each (b,h) is split into.
enum FwdKernel { FK_EMPTY, FK_SHORT, FK_ISO, FK_ISO_PIPE, FK_DIAG_PIPE, FK_DIAG_CHUNK };

FwdKernel pick_kernel(const klaDims* d, int* n_vtiles) {
    const int nvt_env = env_vtiles();
    if (d->T == 0) {
        *n_vtiles = 1;
        return FK_EMPTY;
    }
    if (use_short() && kla::fwd_short_supported(d->dk, d->dv, d->T)) {
        *n_vtiles = 1;
        return FK_SHORT;
    }
    if (d->cov == KLA_ISO) {
        const int nvt_pipe = nvt_env > 0 ? nvt_env : kla::fwd_iso_pipe_vtiles(d->B, d->H, d->dk, d->dv);
        if (use_iso_pipe() && nvt_pipe > 0 &&
            kla::fwd_iso_pipe_supported(d->dk, d->dv, nvt_pipe, d->dtype)) {
            *n_vtiles = nvt_pipe;
            return FK_ISO_PIPE;
        }
        *n_vtiles = nvt_env > 0 ? nvt_env : kla::fwd_iso_vtiles(d->B, d->H, d->dk);
        return FK_ISO;
    }
    if (use_pipe()) {
        const int nvt_pipe = nvt_env > 0 ? nvt_env : diag_pipe_vtiles(d);
        if (nvt_pipe > 0 && kla::fwd_diag_pipe_supported(d->dk, d->dv, nvt_pipe, d->dtype)) {
            *n_vtiles = nvt_pipe;
            return FK_DIAG_PIPE;
        }
    }
    *n_vtiles = nvt_env > 0 ? nvt_env : kla::fwd_diag_vtiles(d->B, d->H, d->T, d->dk, d->dv);
    return FK_DIAG_CHUNK;
}

// Sequence segments klaFwd uses for these dims (1 = no split) and their
// length: segments of seg_len tokens, the last one ragged and non-empty.
// nvt_run: the value tiles the caller launches with, if it picks them itself
// (the block prologue keeps 64-column tiles); 0 = those of pick_kernel.
int pick_nseg(const klaDims* d, int* seg_len = nullptr, int nvt_run = 0) {
    int nvt = 1;
    if (d->T <= 0 || pick_kernel(d, &nvt) != FK_DIAG_PIPE) return 1;
    if (nvt_run > 0) nvt = nvt_run;
    const int e = env_nseg();
    int n = e > 0 ? e : kla::fwd_diag_nseg(d->B, d->H, d->T, d->dk, d->dv, nvt);
    if (n <= 1) return 1;
    const int len = kla::fwd_diag_seg_len(d->T, n);
    n = (d->T + len - 1) / len;
    if (seg_len) *seg_len = len;
    return n < 1 ? 1 : n;
}

size_t seg_bytes(const klaDims* d, int nseg) {
    if (nseg <= 1) return 0;
    return kla::seg_workspace(d->B, d->H, d->T, d->dk, d->dv, d->dtype == KLA_BF16 ? 2 : 4, nseg).bytes;
}

}  // namespace

extern "C" {

const char* klaFwdKernelName(const klaDims* d) {
    if (!d || !dims_ok(d) || !supported(d)) return "";
    int nvt = 1;
    switch (pick_kernel(d, &nvt)) {
        case FK_EMPTY: return "kla_fwd_empty_kernel";
        case FK_SHORT: return "kla_fwd_short_kernel";
        case FK_ISO: return nvt > 1 ? "kla_fwd_iso_kernel (value tiles)" : "kla_fwd_iso_kernel";
        case FK_ISO_PIPE:
            return nvt > 1 ? "kla_fwd_iso_pipe_kernel (value tiles)" : "kla_fwd_iso_pipe_kernel";
        case FK_DIAG_PIPE:
            return nvt > 1 ? "kla_fwd_diag_pipe_kernel (value tiles)" : "kla_fwd_diag_pipe_kernel";
        default: return nvt > 1 ? "kla_fwd_diag_kernel (value tiles)" : "kla_fwd_diag_kernel";
    }
}

int klaIsSupported(const klaDims* d) {
    if (!d || !dims_ok(d)) return 0;
    return supported(d) && kla::step_supported(d->dk, d->dv, d->dtype, d->cov) ? 1 : 0;
}

size_t klaFwdWorkspaceBytes(const klaDims* d) {
    if (!d || !dims_ok(d) || !supported(d) || d->B == 0 || d->H == 0) return 0;
    return seg_bytes(d, pick_nseg(d));
}

}  // extern "C"

namespace {

// The wave-specialised diagonal forward, split into sequence segments when
// pick_nseg says so: precision warm-up (exact segment products and precision
// carry where it did not settle), segment forwards, state carry, output
// correction.  workspace holds klaFwdWorkspaceBytes(d) bytes when split.
hipError_t launch_diag_pipe(kla::FwdArgs& fa, const klaDims* d, void* workspace, hipStream_t st) {
    int seg_len = 0;
    const int nseg = pick_nseg(d, &seg_len, fa.n_vtiles);
    if (nseg <= 1) return kla::launch_fwd_diag_pipe(fa, d->dtype, st);
    const size_t es = d->dtype == KLA_BF16 ? 2 : 4;
    const kla::SegWorkspace w = kla::seg_workspace(d->B, d->H, d->T, d->dk, d->dv, (int)es, nseg);
    char* ws = (char*)workspace;
    float* P = (float*)(ws + w.off_P);
    fa.nseg = nseg;
    fa.seg_len = seg_len;
    fa.seg_l0 = (const float*)(ws + w.off_l0);
    fa.seg_d = (float*)(ws + w.off_d);
    fa.seg_lend = (float*)(ws + w.off_lend);
    fa.seg_m = (float*)(ws + w.off_m);
    fa.seg_qhat = ws + w.off_qhat;
    int* ok = (int*)(ws + w.off_ok);
    hipError_t e = kla::launch_seg_warm(fa, ok, d->dtype, st);
    if (e == hipSuccess) e = kla::launch_seg_mobius(fa, P, ok, d->dtype, st);
    if (e == hipSuccess) e = kla::launch_fwd_diag_pipe(fa, d->dtype, st);
    if (e == hipSuccess) e = kla::launch_seg_carry_m(fa, st);
    if (e == hipSuccess) e = kla::launch_seg_correct(fa, d->dtype, st);
    return e;
}

// klaFwd, or (scratch) klaFwdNoAlloc: the split workspace is then the
// library's device scratch, looked up after every host check has passed.
klaStatus fwd_entry(const klaDims* d, const void* q, const void* k, const void* v, const float* a,
                    const float* qnoise, const float* r, const float* l0, const float* eta0, void* o,
                    float* lT, float* etaT, void* workspace, size_t workspaceBytes, void* hipStream,
                    bool scratch) {
    if (!d) return KLA_ERR_NULL;
    if (!dims_ok(d)) return KLA_ERR_SHAPE;
    if (!kinds_ok(d) || !supported(d)) return KLA_ERR_UNSUPPORTED;
    const long long B = d->B, H = d->H, T = d->T, dk = d->dk, dv = d->dv;
    const long long BH = B * H;
    if (BH > (1LL << 30) || T > (1LL << 30)) return KLA_ERR_SHAPE;
    const bool iso = d->cov == KLA_ISO;
    const size_t es = d->dtype == KLA_BF16 ? 2 : 4;
    const size_t nlt = (size_t)(iso ? BH : BH * dk);
    const size_t neta = (size_t)(BH * dk * dv);

    if (BH == 0) return KLA_OK;
    const bool has_tokens = T > 0;
    // With T == 0 no token input is read; only the state is passed through.
    if (has_tokens && (!q || !k || !v || !a || !qnoise || !r || !o)) return KLA_ERR_NULL;

    const void* big[] = {q, k, v, a, o, eta0, etaT, qnoise, r, l0, lT};
    for (const void* p : big)
        if (p && !aligned16(p)) return KLA_ERR_ALIGN;

    const size_t wneed = klaFwdWorkspaceBytes(d);
    if (scratch) {
        if (wneed > kla::kNoAllocScratchBytes) return KLA_ERR_WORKSPACE;
    } else {
        if (wneed > 0 && (!workspace || workspaceBytes < wneed)) return KLA_ERR_WORKSPACE;
        if (wneed > 0 && !aligned16(workspace)) return KLA_ERR_ALIGN;
    }

    const size_t ntk = (size_t)(BH * T);
    const Span s_o = span(o, ntk * dv * es);
    const Span s_lT = span(lT, nlt * 4), s_etaT = span(etaT, neta * 4);
    const Span ins[] = {span(q, ntk * dk * es), span(k, ntk * dk * es), span(v, ntk * dv * es),
                        span(a, (iso ? ntk : ntk * dk) * 4),
                        span(qnoise, (iso ? ntk : (size_t)(H * dk)) * 4), span(r, ntk * 4),
                        span(l0, nlt * 4), span(eta0, neta * 4)};
    for (const Span& s : ins) {
        if (overlap(s_o, s) || overlap(s_lT, s) || overlap(s_etaT, s)) return KLA_ERR_ALIAS;
    }
    if (overlap(s_o, s_lT) || overlap(s_o, s_etaT) || overlap(s_lT, s_etaT)) return KLA_ERR_ALIAS;
    if (wneed > 0 && !scratch) {
        const Span s_ws = span(workspace, wneed);
        for (const Span& s : ins)
            if (overlap(s_ws, s)) return KLA_ERR_ALIAS;
        if (overlap(s_ws, s_o) || overlap(s_ws, s_lT) || overlap(s_ws, s_etaT)) return KLA_ERR_ALIAS;
    }

    if (scratch && wneed > 0) {
        // the static device array stands in for the caller's workspace
        if (kla::noalloc_scratch(&workspace) != hipSuccess) return KLA_ERR_HIP;
    }

    kla::FwdArgs fa;
    fa.q = q; fa.k = k; fa.v = v; fa.a = a; fa.qn = qnoise; fa.r = r;
    fa.l0 = l0; fa.eta0 = eta0; fa.o = o; fa.lT = lT; fa.etaT = etaT;
    fa.B = (int)B; fa.H = (int)H; fa.T = (int)T; fa.dk = (int)dk; fa.dv = (int)dv;
    fa.chain_scan = use_chain_scan();
    hipStream_t st = (hipStream_t)hipStream;

    hipError_t e;
    switch (pick_kernel(d, &fa.n_vtiles)) {
        case FK_EMPTY: e = kla::launch_fwd_empty(fa, iso ? 1 : 0, st); break;
        case FK_SHORT: e = kla::launch_fwd_short(fa, d->dtype, iso ? 1 : 0, st); break;
        case FK_ISO:
            if (fa.dv % fa.n_vtiles) return KLA_ERR_UNSUPPORTED;
            e = kla::launch_fwd_iso(fa, d->dtype, st);
            break;
        case FK_ISO_PIPE: e = kla::launch_fwd_iso_pipe(fa, d->dtype, st); break;
        case FK_DIAG_PIPE: e = launch_diag_pipe(fa, d, workspace, st); break;
        default: e = kla::launch_fwd_diag(fa, d->dtype, st); break;
    }
    if (e == hipErrorInvalidValue) return KLA_ERR_UNSUPPORTED;
    return e == hipSuccess ? KLA_OK : KLA_ERR_HIP;
}

}  // namespace

extern "C" {

klaStatus klaFwd(const klaDims* d, const void* q, const void* k, const void* v, const float* a,
                 const float* qnoise, const float* r, const float* l0, const float* eta0, void* o,
                 float* lT, float* etaT, void* workspace, size_t workspaceBytes, void* hipStream) {
    return fwd_entry(d, q, k, v, a, qnoise, r, l0, eta0, o, lT, etaT, workspace, workspaceBytes,
                     hipStream, false);
}

klaStatus klaFwdNoAlloc(const klaDims* d, const void* q, const void* k, const void* v, const float* a,
                        const float* qnoise, const float* r, const float* l0, const float* eta0,
                        void* o, float* lT, float* etaT, void* hipStream) {
    return fwd_entry(d, q, k, v, a, qnoise, r, l0, eta0, o, lT, etaT, nullptr, 0, hipStream, true);
}

klaStatus klaFwdBlock(const klaDims* d, const klaBlock* blk, const void* xq, const void* xk, const void* xv,
                      const void* za, const float* zqn, const float* zr, const float* l0, const float* eta0,
                      void* o, float* lT, float* etaT, void* workspace, size_t workspaceBytes,
                      void* hipStream) {
    if (!d || !blk) return KLA_ERR_NULL;
    if (!dims_ok(d)) return KLA_ERR_SHAPE;
    if (!kinds_ok(d) || d->cov != KLA_DIAG) return KLA_ERR_UNSUPPORTED;
    const int nvt = kla::fwd_diag_pipe_vtiles(d->dk, d->dv, d->dtype);
    if (nvt <= 0) return KLA_ERR_UNSUPPORTED;
    const int W = blk->width;
    if (W < 1 || W > 4 || !(blk->r_eps >= 0.f)) return KLA_ERR_SHAPE;
    const long long B = d->B, H = d->H, T = d->T, dk = d->dk, dv = d->dv;
    const long long BH = B * H;
    if (BH > (1LL << 30) || T > (1LL << 30)) return KLA_ERR_SHAPE;
    if (BH == 0) return KLA_OK;
    const size_t es = d->dtype == KLA_BF16 ? 2 : 4;
    if (T > 0 && (!xq || !xk || !xv || !za || !zqn || !zr || !o || !blk->wq || !blk->wk || !blk->wv))
        return KLA_ERR_NULL;
    const void* big[] = {xq, xk, xv, za, o, eta0, etaT, zqn, zr, l0, lT, blk->sq, blk->sk, blk->sv};
    for (const void* p : big)
        if (p && !aligned16(p)) return KLA_ERR_ALIGN;
    const void* small[] = {blk->wq, blk->wk, blk->wv, blk->bq, blk->bk, blk->bv};
    for (const void* p : small)
        if (((uintptr_t)p & 3u) != 0) return KLA_ERR_ALIGN;
    // the sequence split of few, long sequences, as for klaFwd
    const size_t wneed = klaFwdWorkspaceBytes(d);
    if (wneed > 0 && (!workspace || workspaceBytes < wneed)) return KLA_ERR_WORKSPACE;
    if (wneed > 0 && !aligned16(workspace)) return KLA_ERR_ALIGN;

    const size_t ntk = (size_t)(BH * T), nlt = (size_t)(BH * dk), neta = (size_t)(BH * dk * dv);
    const Span s_o = span(o, ntk * dv * es);
    const Span s_lT = span(lT, nlt * 4), s_etaT = span(etaT, neta * 4);
    const size_t ws = (size_t)(W - 1);
    const Span ins[] = {span(xq, ntk * dk * es), span(xk, ntk * dk * es), span(xv, ntk * dv * es),
                        span(za, ntk * dk * es), span(zqn, (size_t)(H * dk) * 4), span(zr, ntk * 4),
                        span(l0, nlt * 4), span(eta0, neta * 4),
                        span(blk->wq, (size_t)(H * dk) * W * 4), span(blk->wk, (size_t)(H * dk) * W * 4),
                        span(blk->wv, (size_t)(H * dv) * W * 4), span(blk->bq, (size_t)(H * dk) * 4),
                        span(blk->bk, (size_t)(H * dk) * 4), span(blk->bv, (size_t)(H * dv) * 4),
                        span(blk->sq, (size_t)BH * ws * dk * es), span(blk->sk, (size_t)BH * ws * dk * es),
                        span(blk->sv, (size_t)BH * ws * dv * es)};
    for (const Span& s : ins)
        if (overlap(s_o, s) || overlap(s_lT, s) || overlap(s_etaT, s)) return KLA_ERR_ALIAS;
    if (overlap(s_o, s_lT) || overlap(s_o, s_etaT) || overlap(s_lT, s_etaT)) return KLA_ERR_ALIAS;
    if (wneed > 0) {
        const Span s_ws = span(workspace, wneed);
        for (const Span& s : ins)
            if (overlap(s_ws, s)) return KLA_ERR_ALIAS;
        if (overlap(s_ws, s_o) || overlap(s_ws, s_lT) || overlap(s_ws, s_etaT)) return KLA_ERR_ALIAS;
    }

    kla::FwdArgs fa;
    fa.q = xq; fa.k = xk; fa.v = xv; fa.a = (const float*)za; fa.qn = zqn; fa.r = zr;
    fa.l0 = l0; fa.eta0 = eta0; fa.o = o; fa.lT = lT; fa.etaT = etaT;
    fa.B = (int)B; fa.H = (int)H; fa.T = (int)T; fa.dk = (int)dk; fa.dv = (int)dv;
    fa.n_vtiles = nvt;
    fa.conv_w = W;
    fa.conv_wt[0] = blk->wq; fa.conv_wt[1] = blk->wk; fa.conv_wt[2] = blk->wv;
    fa.conv_b[0] = blk->bq; fa.conv_b[1] = blk->bk; fa.conv_b[2] = blk->bv;
    fa.conv_s[0] = blk->sq; fa.conv_s[1] = blk->sk; fa.conv_s[2] = blk->sv;
    fa.r_eps = blk->r_eps;
    hipStream_t st = (hipStream_t)hipStream;
    const hipError_t e = T == 0 ? kla::launch_fwd_empty(fa, 0, st) : launch_diag_pipe(fa, d, workspace, st);
    if (e == hipErrorInvalidValue) return KLA_ERR_UNSUPPORTED;
    return e == hipSuccess ? KLA_OK : KLA_ERR_HIP;
}

klaStatus klaStep(const klaDims* d, const void* q, const void* k, const void* v, const float* a,
                  const float* qnoise, const float* r, float* l, float* eta, void* o,
                  void* hipStream) {
    if (!d) return KLA_ERR_NULL;
    if (d->B < 0 || d->H < 0 || d->dk < 1 || d->dv < 1) return KLA_ERR_SHAPE;
    if (!kinds_ok(d) || !kla::step_supported(d->dk, d->dv, d->dtype, d->cov)) return KLA_ERR_UNSUPPORTED;
    const long long BH = (long long)d->B * d->H;
    if (BH > (1LL << 30)) return KLA_ERR_SHAPE;
    if (BH == 0) return KLA_OK;
    if (!q || !k || !v || !a || !qnoise || !r || !l || !eta || !o) return KLA_ERR_NULL;
    const void* ptrs[] = {q, k, v, a, qnoise, r, l, eta, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return KLA_ERR_ALIGN;
    const bool iso = d->cov == KLA_ISO;
    const size_t es = d->dtype == KLA_BF16 ? 2 : 4;
    const size_t nl = (size_t)(iso ? BH : BH * d->dk);
    const Span s_o = span(o, (size_t)BH * d->dv * es);
    const Span others[] = {span(q, (size_t)BH * d->dk * es), span(k, (size_t)BH * d->dk * es),
                           span(v, (size_t)BH * d->dv * es), span(a, nl * 4),
                           span(qnoise, (iso ? (size_t)BH : (size_t)d->H * d->dk) * 4),
                           span(r, (size_t)BH * 4), span(l, nl * 4),
                           span(eta, (size_t)BH * d->dk * d->dv * 4)};
    for (const Span& s : others)
        if (overlap(s_o, s)) return KLA_ERR_ALIAS;
    if (overlap(span(l, nl * 4), span(eta, (size_t)BH * d->dk * d->dv * 4))) return KLA_ERR_ALIAS;

    kla::StepArgs sa;
    sa.q = q; sa.k = k; sa.v = v; sa.a = a; sa.qn = qnoise; sa.r = r;
    sa.l = l; sa.eta = eta; sa.o = o;
    sa.B = d->B; sa.H = d->H; sa.dk = d->dk; sa.dv = d->dv;
    const hipError_t e = kla::launch_step(sa, d->dtype, d->cov, (hipStream_t)hipStream);
    if (e == hipErrorInvalidValue) return KLA_ERR_UNSUPPORTED;
    return e == hipSuccess ? KLA_OK : KLA_ERR_HIP;
}

const char* klaStatusString(klaStatus s) {
    switch (s) {
        case KLA_OK: return "KLA_OK: success";
        case KLA_ERR_NULL: return "KLA_ERR_NULL: a required pointer is NULL";
        case KLA_ERR_SHAPE: return "KLA_ERR_SHAPE: a dimension is negative or too large";
        case KLA_ERR_UNSUPPORTED: return "KLA_ERR_UNSUPPORTED: (dk, dv, dtype, cov) not built";
        case KLA_ERR_ALIGN: return "KLA_ERR_ALIGN: a pointer is not 16-byte aligned";
        case KLA_ERR_WORKSPACE: return "KLA_ERR_WORKSPACE: workspace missing or too small";
        case KLA_ERR_HIP: return "KLA_ERR_HIP: the HIP runtime reported a launch error";
        case KLA_ERR_INTERNAL: return "KLA_ERR_INTERNAL: internal error";
        case KLA_ERR_ALIAS: return "KLA_ERR_ALIAS: an output overlaps an input";
    }
    return "unknown klaStatus";
}

klaStatus klaFwdResidual(const klaDims* d, const void* q, const void* k, const void* v, const float* a,
                         const float* qnoise, const float* r, const float* l0, const float* m0, void* o,
                         float* lT, float* mT, void* hipStream) {
    if (!d) return KLA_ERR_NULL;
    if (!dims_ok(d)) return KLA_ERR_SHAPE;
    if (!kinds_ok(d) || !kla::fwd_residual_supported(d->dk, d->dv)) return KLA_ERR_UNSUPPORTED;
    const long long B = d->B, H = d->H, T = d->T, dk = d->dk, dv = d->dv;
    const long long BH = B * H;
    if (BH > (1LL << 30) || T > (1LL << 30)) return KLA_ERR_SHAPE;
    const bool iso = d->cov == KLA_ISO;
    const size_t es = d->dtype == KLA_BF16 ? 2 : 4;
    const size_t nlt = (size_t)(iso ? BH : BH * dk);
    const size_t nm = (size_t)(BH * dk * dv);

    if (BH == 0) return KLA_OK;
    if (T > 0 && (!q || !k || !v || !a || !qnoise || !r || !o)) return KLA_ERR_NULL;
    const void* ptrs[] = {q, k, v, a, o, m0, mT, qnoise, r, l0, lT};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KLA_ERR_ALIGN;

    const size_t ntk = (size_t)(BH * T);
    const Span s_o = span(o, ntk * dv * es);
    const Span s_lT = span(lT, nlt * 4), s_mT = span(mT, nm * 4);
    const Span ins[] = {span(q, ntk * dk * es), span(k, ntk * dk * es), span(v, ntk * dv * es),
                        span(a, (iso ? ntk : ntk * dk) * 4),
                        span(qnoise, (iso ? ntk : (size_t)(H * dk)) * 4), span(r, ntk * 4),
                        span(l0, nlt * 4), span(m0, nm * 4)};
    for (const Span& s : ins)
        if (overlap(s_o, s) || overlap(s_lT, s) || overlap(s_mT, s)) return KLA_ERR_ALIAS;
    if (overlap(s_o, s_lT) || overlap(s_o, s_mT) || overlap(s_lT, s_mT)) return KLA_ERR_ALIAS;

    kla::FwdArgs fa;
    fa.q = q; fa.k = k; fa.v = v; fa.a = a; fa.qn = qnoise; fa.r = r;
    fa.l0 = l0; fa.eta0 = m0; fa.o = o; fa.lT = lT; fa.etaT = mT;
    fa.B = (int)B; fa.H = (int)H; fa.T = (int)T; fa.dk = (int)dk; fa.dv = (int)dv;
    fa.n_vtiles = kla::fwd_residual_vtiles(fa.B, fa.H, fa.dk);
    if (const char* env = getenv("KLA_RES_VTILES")) fa.n_vtiles = atoi(env) == 2 && dk >= 64 ? 2 : 1;
    hipStream_t st = (hipStream_t)hipStream;
    const hipError_t e = T == 0 ? kla::launch_fwd_empty(fa, iso ? 1 : 0, st)
                                : kla::launch_fwd_residual(fa, d->dtype, iso ? 1 : 0, st);
    return e == hipSuccess ? KLA_OK : KLA_ERR_HIP;
}

size_t klaBwdWorkspaceBytes(const klaDims* d) {
    if (!d || !dims_ok(d) || !kinds_ok(d) || !kla::bwd_supported(d->dk, d->dv)) return 0;
    return (size_t)d->B * d->H * kla::bwd_ws_stride(d->B, d->H, d->T, d->dk, d->cov == KLA_ISO ? 1 : 0,
                                                            d->dtype == KLA_BF16 ? kla::DT_BF16 : kla::DT_F32) * sizeof(float);
}

klaStatus klaBwd(const klaDims* d, const void* q, const void* k, const void* v, const float* a,
                 const float* qnoise, const float* r, const float* l0, const float* eta0, const void* dO,
                 const float* dlT, const float* detaT, void* dq, void* dk, void* dv, float* da,
                 float* dqnoise, float* dr, float* dl0, float* deta0, void* workspace,
                 size_t workspaceBytes, void* hipStream) {
    if (!d) return KLA_ERR_NULL;
    if (!dims_ok(d)) return KLA_ERR_SHAPE;
    if (!kinds_ok(d) || !kla::bwd_supported(d->dk, d->dv)) return KLA_ERR_UNSUPPORTED;
    const long long B = d->B, H = d->H, T = d->T, dkd = d->dk, dvd = d->dv;
    const long long BH = B * H;
    if (BH > (1LL << 30) || T > (1LL << 30)) return KLA_ERR_SHAPE;
    const bool iso = d->cov == KLA_ISO;
    const size_t es = d->dtype == KLA_BF16 ? 2 : 4;
    const size_t ntk = (size_t)(BH * T);
    const size_t nl = (size_t)(iso ? BH : BH * dkd);
    const size_t neta = (size_t)(BH * dkd * dvd);
    const size_t nqn = iso ? ntk : (size_t)(H * dkd);
    if (H * dkd == 0 || (iso && BH == 0)) return KLA_OK;
    if (!iso && !dqnoise) return KLA_ERR_NULL;
    if (ntk > 0 && (!q || !k || !v || !a || !qnoise || !r || !dO || !dq || !dk || !dv || !da ||
                    !dqnoise || !dr))
        return KLA_ERR_NULL;
    const void* ptrs[] = {q, k, v, a, qnoise, r, l0, eta0, dO, dlT, detaT,
                          dq, dk, dv, da, dqnoise, dr, dl0, deta0};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KLA_ERR_ALIGN;
    const size_t wneed = klaBwdWorkspaceBytes(d);
    if (wneed > 0 && (!workspace || workspaceBytes < wneed)) return KLA_ERR_WORKSPACE;
    if (wneed > 0 && !aligned16(workspace)) return KLA_ERR_ALIGN;
    const Span ins[] = {span(q, ntk * dkd * es), span(k, ntk * dkd * es), span(v, ntk * dvd * es),
                        span(a, (iso ? ntk : ntk * dkd) * 4), span(qnoise, (iso ? ntk : (size_t)(H * dkd)) * 4),
                        span(r, ntk * 4), span(l0, nl * 4), span(eta0, neta * 4),
                        span(dO, ntk * dvd * es), span(dlT, nl * 4), span(detaT, neta * 4)};
    const Span outs[] = {span(dq, ntk * dkd * es), span(dk, ntk * dkd * es), span(dv, ntk * dvd * es),
                         span(da, (iso ? ntk : ntk * dkd) * 4), span(dqnoise, nqn * 4), span(dr, ntk * 4),
                         span(dl0, nl * 4), span(deta0, neta * 4), span(workspace, wneed)};
    const int nout = sizeof(outs) / sizeof(outs[0]);
    for (int x = 0; x < nout; ++x) {
        for (const Span& s : ins)
            if (overlap(outs[x], s)) return KLA_ERR_ALIAS;
        for (int y = x + 1; y < nout; ++y)
            if (overlap(outs[x], outs[y])) return KLA_ERR_ALIAS;
    }
    kla::BwdArgs ba;
    ba.q = q; ba.k = k; ba.v = v; ba.a = a; ba.qn = qnoise; ba.r = r; ba.l0 = l0; ba.eta0 = eta0;
    ba.dO = dO; ba.dlT = dlT; ba.detaT = detaT;
    ba.gq = dq; ba.gk = dk; ba.gv = dv; ba.ga = da; ba.gqn = dqnoise; ba.gr = dr; ba.gl0 = dl0;
    ba.geta0 = deta0;
    ba.ws = (float*)workspace;
    ba.ws_stride = kla::bwd_ws_stride(d->B, d->H, d->T, d->dk, iso ? 1 : 0,
                                     d->dtype == KLA_BF16 ? kla::DT_BF16 : kla::DT_F32);
    ba.gate_nt = 0;
    ba.flag_off = 0;
    ba.spin = 1 << 20;
    ba.B = d->B; ba.H = d->H; ba.T = d->T; ba.dk = d->dk; ba.dv = d->dv;
    const hipError_t e = kla::launch_bwd(ba, d->dtype, iso ? 1 : 0, (hipStream_t)hipStream);
    if (e == hipErrorInvalidValue) return KLA_ERR_UNSUPPORTED;
    return e == hipSuccess ? KLA_OK : KLA_ERR_HIP;
}

}  // extern "C"
