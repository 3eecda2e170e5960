/*
 * kla.h -- C ABI of the MI355X (gfx950) Kalman Linear Attention forward path.
 *
 * Method sources (cited by title and section):
 *  [KLA]  "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
 *         Language Modelling and State Tracking" -- gist.science explainer,
 *         technical summary (技術要約) > method (手法) §1 probabilistic
 *         formulation, §2 Mobius parallelisation, §3 uncertainty gating,
 *         §4 architecture (drop-in replacement for an SSM / attention layer).
 *  [KDN]  "Kalman Delta Networks: Uncertainty-aware Associative Memory" --
 *         abstract: diagonal and isotropic scan-compatible variants and
 *         constant-memory decoding.
 *
 * The operation (per batch b, head h).  The memory is the information form of
 * a Kalman filter over a linear-Gaussian state-space model ([KLA] method §1):
 * OU decay a_t, process noise qn, observation of the value through the key
 * k_t with noise r_t, readout of the posterior mean through the query q_t.
 * The pages fix the Mobius form of the precision map ([KLA] method §2) but not
 * its coefficients; this library computes, for every key dim i,
 *
 *   lp          = l_{t-1}[i] / (a_t[i]^2 + qn[i] * l_{t-1}[i])
 *   l_t[i]      = lp + k_t[i]^2 / r_t
 *   eta_t[i,:]  = (lp * a_t[i] / l_{t-1}[i]) * eta_{t-1}[i,:] + k_t[i] v_t / r_t
 *   o_t         = sum_i q_t[i] * eta_t[i,:] / l_t[i]
 *
 * i.e. the precision map l -> ((1 + b qn) l + b a^2) / (qn l + a^2) with
 * b = k^2 / r, composed associatively as 2x2 projective matrices.  In the
 * isotropic variant ([KDN]) l is one scalar per head, a_t and qn_t are per
 * token, and the precision increment is b_t = sum_i k_t[i]^2 / (d_k r_t);
 * the information rows are updated as above with the scalar gate.
 * klaFwdResidual (below) computes the residual-write variant of [KDN], in
 * which the key dims are coupled through the prediction of v.
 * (Short sequences and decode steps continue a cached state; see klaFwd and
 * klaStep.)
 *
 * Layouts: dense, row-major, head-major ("BHTD"):
 *   q, k        [B,H,T,dk]      dtype (fp32 or bf16)
 *   v, o        [B,H,T,dv]      dtype
 *   r           [B,H,T]         fp32
 *   diag:  a [B,H,T,dk]  qn [H,dk]    l0,lT [B,H,dk]   fp32
 *   iso:   a [B,H,T]     qn [B,H,T]   l0,lT [B,H]      fp32
 *   eta0, etaT  [B,H,dk,dv]     fp32
 *
 * Ownership and execution: every pointer is a DEVICE pointer owned by the
 * caller.  The library never allocates, frees or synchronises device
 * memory; all work is enqueued asynchronously on the given HIP stream
 * (NULL = the default stream).  Outputs are fully overwritten.  The library
 * holds no mutable global state and is reentrant.
 *
 * Errors: argument errors are detected on the host and returned before any
 * HIP call, with nothing written.  A failing launch returns KLA_ERR_HIP.
 * No C++ exception crosses this interface.
 *
 * Numerical preconditions (documented, not checked on the device):
 * r > 0, l0 > 0, 0 < a <= 1, qn >= 0, a^2 + qn * l > 0.  Otherwise the
 * results are undefined (they propagate as NaN/Inf).  With qn = 0 and a < 1
 * the precision grows by 1/a^2 per token and leaves the fp32 range after
 * about 64 / |log2 a| tokens; the results are then Inf/NaN as well.
 */
#ifndef KLA_H
#define KLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KLA_OK = 0,
    KLA_ERR_NULL = 1,        /* a required pointer is NULL                         */
    KLA_ERR_SHAPE = 2,       /* a dimension is negative or the dims pointer is bad */
    KLA_ERR_UNSUPPORTED = 3, /* (dk, dv, dtype, cov) combination not built          */
    KLA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                    */
    KLA_ERR_WORKSPACE = 5,   /* workspace smaller than klaFwdWorkspaceBytes()       */
    KLA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch         */
    KLA_ERR_INTERNAL = 7,    /* unexpected internal condition                       */
    KLA_ERR_ALIAS = 8        /* an output overlaps an input it must not overlap     */
} klaStatus;

typedef enum { KLA_F32 = 0, KLA_BF16 = 1 } klaDtype; /* dtype of q, k, v and o */
typedef enum { KLA_DIAG = 0, KLA_ISO = 1 } klaCov;   /* precision structure   */

typedef struct {
    int B, H, T;  /* batch, heads, tokens (T is ignored by klaStep)          */
    int dk, dv;   /* key and value head dims                                 */
    int dtype;    /* klaDtype                                                */
    int cov;      /* klaCov                                                  */
} klaDims;

/* Whether klaFwd/klaStep accept these dims (dk, dv, dtype, cov). */
int klaIsSupported(const klaDims* d);

/*
 * Device workspace (bytes) that klaFwd needs for these dims; 0 means none
 * (workspace may then be NULL).  Returns 0 for unsupported dims too.
 * Long sequences are split across workgroups and their carries pass through
 * the workspace.
 */
size_t klaFwdWorkspaceBytes(const klaDims* d);

/*
 * Forward pass over T tokens for all (b,h) ([KLA] method §1-§3; [KDN]).
 * In:  q, k, v, a, qnoise, r as laid out above; l0, eta0 the filter state
 *      before the first token (l0 == NULL means l0 = 1; eta0 == NULL means
 *      eta0 = 0; they are independent).
 * Out: o [B,H,T,dv] (o_t uses the posterior after token t); lT, etaT the
 *      state after the last token (either may be NULL to skip it).
 * T == 0 (or B*H == 0) is valid: o is empty and lT/etaT receive l0/eta0;
 * the token inputs (q, k, v, a, qnoise, r, o) may then be NULL.
 * Every non-NULL pointer must be 16-byte aligned (KLA_ERR_ALIGN).
 * Aliasing: o must not overlap any input; lT/etaT must not overlap l0/eta0
 * (KLA_ERR_ALIAS).  workspace must hold klaFwdWorkspaceBytes(d) bytes and
 * must not be used by another call that runs at the same time.
 * Serving: a prefill chunk or several decode tokens continue a cached state
 * by passing it as l0/eta0 and a second state buffer as lT/etaT (constant-
 * memory decoding, [KDN]); up to 32 tokens run on a kernel that holds the
 * state on chip for the whole call.
 */
klaStatus klaFwd(const klaDims* d,
                 const void* q, const void* k, const void* v,
                 const float* a, const float* qnoise, const float* r,
                 const float* l0, const float* eta0,
                 void* o, float* lT, float* etaT,
                 void* workspace, size_t workspaceBytes, void* hipStream);

/*
 * klaFwd for callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, results
 * and errors as klaFwd, without the workspace: when the call needs one
 * (klaFwdWorkspaceBytes(d) > 0, the sequence split of few, long diagonal
 * sequences) it uses a device array of the library, 64 MiB per GPU, held from
 * the library's load until the process ends.  A call that needs more returns
 * KLA_ERR_WORKSPACE before any HIP call.  No memory is allocated or freed.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (several streams or host threads) race and must be serialised by the
 * caller.
 */
klaStatus klaFwdNoAlloc(const klaDims* d,
                        const void* q, const void* k, const void* v,
                        const float* a, const float* qnoise, const float* r,
                        const float* l0, const float* eta0,
                        void* o, float* lT, float* etaT, void* hipStream);

/*
 * Fused block prologue.  "Kalman Linear Attention: Parallel Bayesian
 * Filtering For Efficient Language Modelling and State Tracking" (gist.science
 * explainer, technical summary > method §4, architecture): the layer is a
 * Mamba-like fused block with a one-dimensional causal convolution and SiLU.
 * klaFwdBlock runs the diagonal forward with that prologue inside its loads:
 *   q = silu(conv_q(xq)), k = silu(conv_k(xk)), v = silu(conv_v(xv)),
 *   a = sigmoid(za), qn = softplus(zqn), r = softplus(zr) + r_eps,
 * where conv_x is a depthwise causal convolution of `width` taps along the
 * sequence: conv(x)_t[c] = bias[c] + sum_{j<W} w[c][W-1-j] x_{t-j}[c] (tap
 * W-1 on the current token).  Rows before token 0 come from the convolution
 * state (the W-1 preceding rows, oldest first) or are zero.  A chunked
 * prefill continues a sequence by passing the previous chunk's last W-1 rows
 * of xq, xk, xv as the state and its lT, etaT as l0, eta0.
 */
typedef struct klaBlock {
    int width;                         /* W, 1..4                              */
    const float* wq;                   /* taps [H, dk, W] fp32                 */
    const float* wk;                   /* taps [H, dk, W] fp32                 */
    const float* wv;                   /* taps [H, dv, W] fp32                 */
    const float* bq;                   /* biases [H, dk] fp32, or NULL (zero)  */
    const float* bk;                   /* biases [H, dk] fp32, or NULL (zero)  */
    const float* bv;                   /* biases [H, dv] fp32, or NULL (zero)  */
    const void* sq;                    /* states [B, H, W-1, dk] (dtype), or NULL (zero) */
    const void* sk;                    /* states [B, H, W-1, dk] (dtype), or NULL (zero) */
    const void* sv;                    /* states [B, H, W-1, dv] (dtype), or NULL (zero) */
    float r_eps;                       /* r = softplus(zr) + r_eps, r_eps >= 0 */
} klaBlock;

/*
 * In:  xq, xk [B,H,T,dk], xv [B,H,T,dv] and za [B,H,T,dk] in d->dtype;
 *      zqn [H,dk] and zr [B,H,T] fp32; l0, eta0 as for klaFwd (NULL: l0 = 1,
 *      eta0 = 0); blk as above (NULL: KLA_ERR_NULL).
 * Out: o [B,H,T,dv] (dtype), lT, etaT (may be NULL) as for klaFwd.
 * Diagonal covariance only, dk = dv in {64, 128} (128: bf16), the dims of
 * the wave-specialised kernel (KLA_ERR_UNSUPPORTED otherwise); width outside
 * 1..4 or r_eps < 0 is KLA_ERR_SHAPE.  Few, long sequences are split into
 * segments as for klaFwd: workspace must then hold klaFwdWorkspaceBytes(d)
 * bytes (KLA_ERR_WORKSPACE otherwise; NULL when that is 0) and must not be
 * used by another call at the same time.  No memory is allocated.  Every
 * non-NULL pointer must be 16-byte aligned except the taps and biases
 * (4-byte).  o must not overlap an input; lT and etaT must not overlap l0,
 * eta0; the workspace must not overlap any argument (KLA_ERR_ALIAS).
 * T == 0 passes l0/eta0 through.
 */
klaStatus klaFwdBlock(const klaDims* d, const klaBlock* blk,
                      const void* xq, const void* xk, const void* xv,
                      const void* za, const float* zqn, const float* zr,
                      const float* l0, const float* eta0,
                      void* o, float* lT, float* etaT,
                      void* workspace, size_t workspaceBytes, void* hipStream);

/*
 * One decode step for every (b,h) (the same recurrence with T = 1;
 * constant-memory decoding, [KDN]).  State is updated in place.
 * Layouts: q, k [B,H,dk]; v, o [B,H,dv]; r [B,H];
 *          diag: a [B,H,dk], qnoise [H,dk], l [B,H,dk];
 *          iso:  a, qnoise, l [B,H];  eta [B,H,dk,dv] (all fp32 except q,k,v,o).
 * d->T is ignored.  o must not overlap the other arguments.
 */
klaStatus klaStep(const klaDims* d,
                  const void* q, const void* k, const void* v,
                  const float* a, const float* qnoise, const float* r,
                  float* l, float* eta, void* o, void* hipStream);

/*
 * Residual-write forward over T tokens for all (b,h) ([KDN]: the Kalman gain
 * weights each residual write).  The memory is observed through the full key
 * contraction, v_t = x_t^T k_t + noise, and each one-step posterior is
 * projected onto the diagonal (isotropic) Gaussian family by mean-field
 * variational inference, which keeps its mean.  With the state (l, m), m the
 * posterior MEAN [B,H,dk,dv] (not the information l*m of klaFwd):
 *     lp = l / (a^2 + qnoise*l),   m_pred = a (.) m   (row i scaled by a_i)
 *     g  = (k/lp) / (sum_i k_i^2/lp_i + r)            (iso: k / (|k|^2 + r*lp))
 *     m  = m_pred + g (v - m_pred^T k)^T
 *     l  = lp + k^2/r                                  (iso: lp + |k|^2/(dk*r))
 *     o  = m^T q
 * Layouts, dtypes, alignment, ownership and execution as klaFwd, with m0 / mT
 * in place of eta0 / etaT (m0 == NULL means m0 = 0; l0 == NULL means l0 = 1;
 * lT, mT may be NULL).  Supported: dk == dv in {16, 32, 64, 128}, either
 * dtype and cov (KLA_ERR_UNSUPPORTED otherwise); no workspace.  T == 0
 * passes the state through.  Aliasing: o must not overlap any input; lT / mT
 * must not overlap l0 / m0 (KLA_ERR_ALIAS).
 */
klaStatus klaFwdResidual(const klaDims* d,
                         const void* q, const void* k, const void* v,
                         const float* a, const float* qnoise, const float* r,
                         const float* l0, const float* m0,
                         void* o, float* lT, float* mT, void* hipStream);

/*
 * Device workspace (bytes) that klaBwd needs for these dims: per (b,h) the
 * precision after every token and one scalar per token and key dim (per
 * token when isotropic), both fp64, plus dk fp32 for the diagonal, rounded up
 * to 256 bytes per (b,h).  0 for unsupported dims.
 */
size_t klaBwdWorkspaceBytes(const klaDims* d);

/*
 * Backward pass of klaFwd ([KLA] abstract: the information-form filter is
 * trained in parallel as a sequence-model layer, so its gradients are part of
 * the layer).  For the scalar L = <dO, o> + <dlT, lT> + <detaT, etaT> of one
 * klaFwd call with the same inputs, it returns dL/dq, dL/dk, dL/dv, dL/da,
 * dL/dqnoise, dL/dr, dL/dl0 and dL/deta0.
 * In:  q, k, v, a, qnoise, r, l0, eta0 exactly as passed to klaFwd (l0, eta0
 *      may be NULL: 1 and 0); dO [B,H,T,dv] in the input dtype; dlT (shape of
 *      lT) and detaT [B,H,dk,dv] fp32, either may be NULL (zero).
 * Out: dq, dk [B,H,T,dk] and dv [B,H,T,dv] in the input dtype (rounded RNE
 *      from fp32); da (diag [B,H,T,dk], iso [B,H,T]), dr [B,H,T] fp32;
 *      dqnoise fp32: diag [H,dk], summed over the batch; iso [B,H,T];
 *      dl0 (shape of l0) and deta0 [B,H,dk,dv] fp32, either may be NULL
 *      (not computed).  All outputs are fully overwritten.
 * Supported: dk == dv in {16, 32, 64, 128}, either dtype and cov.
 * workspace must hold klaBwdWorkspaceBytes(d) bytes (16-byte aligned).
 * Every non-NULL pointer must be 16-byte aligned.  Aliasing: no output may
 * overlap an input, the workspace or another output (KLA_ERR_ALIAS).
 * Errors, ownership and execution as klaFwd; preconditions as klaFwd, with
 * a > 0 (the gradient of the gate divides by a).
 */
klaStatus klaBwd(const klaDims* d,
                 const void* q, const void* k, const void* v,
                 const float* a, const float* qnoise, const float* r,
                 const float* l0, const float* eta0,
                 const void* dO, const float* dlT, const float* detaT,
                 void* dq, void* dk, void* dv, float* da, float* dqnoise, float* dr,
                 float* dl0, float* deta0,
                 void* workspace, size_t workspaceBytes, void* hipStream);

/* Static, human-readable description of a status code (never NULL). */
const char* klaStatusString(klaStatus s);

/*
 * Diagnostic: name of the kernel family that klaFwd launches for these dims
 * (the name profilers show, e.g. "kla_fwd_diag_pipe_kernel"; " (value tiles)"
 * is appended when each (b,h) is split over several workgroups by value
 * columns).  Static string, never NULL; "" for NULL, invalid or unsupported
 * dims.  Honours the same environment overrides as klaFwd.
 */
const char* klaFwdKernelName(const klaDims* d);

#ifdef __cplusplus
}
#endif

#endif /* KLA_H */
