/*
 * gdr.h -- C ABI of the chunkwise gated delta rule forward pass for MI355X
 * (gfx950).  Plain C: no C++ or torch types cross this boundary.
 *
 * The operation (sec-03 notes "Chunkwise": in-chunk cumsum and triangular
 * solve, code comparison, inter-chunk recurrence; "Chunkwise parallel
 * algorithms" page, sections 2.1-2.4) maps, for every batch b and value head
 * hv with q/k head h = hv / (HV/H),
 *
 *     S <- diag(exp(g_t)) S ;  S <- S + beta_t k_t (v_t - S^T k_t)^T ;
 *     o_t = scale * S^T q_t                            (t = 0 .. T-1)
 *
 * and computes it chunkwise with chunk length C: in-chunk cumsum gamma of g,
 * the decayed dot matrices A_kk and A_qk, the UT transform (the inverse of
 * M = I + strictly_lower(A_kk diag(beta))), and the serial inter-chunk
 * recurrence of the K x V state.  The result equals that recurrence up to
 * floating-point rounding.
 *
 * Tensor layouts (row-major, contiguous, device memory):
 *   q, k           [B, T, H, K]    qkv_dtype (GDR_F32, GDR_BF16 or GDR_F16)
 *   v              [B, T, HV, V]   qkv_dtype
 *   g              [B, T, HV] fp32 (one log-decay per value head), or
 *                  [B, T, HV, K] fp32 when g_per_channel = 1 (KDA form)
 *   beta           [B, T, HV]      fp32
 *   initial_state  [B, HV, K, V]   fp32, or NULL for a zero state
 *   o              [B, T, HV, V]   o_dtype: fp32, bf16 or fp16 (output)
 *   final_state    [B, HV, K, V]   fp32 (output), or NULL to skip
 *
 * Ownership: the caller allocates and owns every buffer, the workspace
 * included.  The library never allocates or frees device memory; its global
 * state is a per-device cache of the architecture check and, for
 * gdr_chunk_fwd_noalloc only, a static device scratch array (one per GPU,
 * held until the process ends) with its per-device address.  Calls on
 * different streams are independent when they use different workspaces and
 * outputs (gdr_chunk_fwd_noalloc calls on one GPU share its scratch array).
 *
 * Streams: work is enqueued asynchronously on `stream` (a hipStream_t; NULL
 * is the null stream).  No call synchronises.  A fault inside a kernel shows
 * up at the caller's next synchronisation.
 *
 * Errors: arguments are validated before any HIP call.  On an error nothing
 * is launched and a status other than GDR_OK is returned; no exception
 * crosses the ABI.  gdr_status_string() names every status.
 *
 * Numerics: with GDR_BF16 or GDR_F16 inputs the matrix products run on
 * MFMA with fp16 operands and fp32 accumulation (fp16 inputs are operands
 * as they are); the state, gamma, exponentials and o are fp32 (o is rounded
 * to bf16 or fp16 only as it is stored, when o_dtype asks).  bf16 inputs
 * must have |x| < 65504 (the fp16 range).  With GDR_F32 inputs every
 * product runs in fp32.  With 16-bit inputs the decay is folded
 * into fp16 operands, which grow as exp(sum of the positive g of a channel,
 * or of the row decay, within one chunk): that sum must stay at or below 8
 * (g <= 0, the usual log-decay, is always in range).  The state enters its
 * products as fp16 too, so its entries must stay below 65504 in magnitude.
 * gdr_check_inputs tests the inputs against these bounds on the device;
 * nothing else checks them, and a violation shows as inf or NaN in o.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdr_status {
  GDR_OK = 0,
  GDR_ERR_NULL = 1,        /* a required pointer (problem, q, k, v, g, beta, o) is NULL */
  GDR_ERR_SHAPE = 2,       /* B, T, H, HV, K or V < 1, or HV % H != 0 */
  GDR_ERR_DTYPE = 3,       /* qkv_dtype or o_dtype is not a gdr_dtype value */
  GDR_ERR_UNSUPPORTED = 4, /* valid but not built: chunk not 0, 32, 64 or 128, K or V
                              not 64 or 128, or a scan_slab the chunk length lacks */
  GDR_ERR_ALIGN = 5,       /* a tensor or workspace pointer is not 16-byte aligned */
  GDR_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the size query */
  GDR_ERR_DEVICE = 7,      /* the current HIP device is not a gfx950 */
  GDR_ERR_HIP = 8,         /* a HIP query or kernel launch failed */
  GDR_ERR_ARG = 9,         /* scale not finite, chunk < 0, g_per_channel or
                              qk_l2norm not 0/1, rule not a gdr_rule,
                              scan_segments < 0, or scan_slab not 0, 32 or 64
                              (gdr_decode_step also takes 128) */
  GDR_ERR_ALIAS = 10,      /* an output overlaps an input or the other output
                              (final_state == initial_state exactly is allowed),
                              or the workspace overlaps an input, a state or o;
                              inputs may overlap each other (they are only read) */
  GDR_ERR_SCRATCH = 11     /* gdr_chunk_fwd_noalloc: the problem needs more
                              workspace than GDR_NOALLOC_SCRATCH_BYTES */
} gdr_status;

/* Bytes of the library's own device scratch array behind
 * gdr_chunk_fwd_noalloc: one array per GPU the library runs on, held until
 * the process ends. */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum gdr_dtype { GDR_F32 = 0, GDR_BF16 = 1, GDR_F16 = 2 } gdr_dtype;

/* The state update.  GDR_RULE_DELTA is the gated delta rule above.
 * GDR_RULE_LINEAR drops its prediction (erase) term,
 *     S <- diag(exp(g_t)) S + beta_t k_t v_t^T,  o_t = scale * S^T q_t,
 * the decayed linear attention of the Mamba2 state-space-duality section of
 * the "Chunkwise parallel algorithms" page (section 1.1; beta = 1 and
 * scale = 1 give its form exactly; per-channel g gives the gated linear
 * attention form).  Its chunk form is the same with M = I: the UT transform
 * drops out. */
typedef enum gdr_rule { GDR_RULE_DELTA = 0, GDR_RULE_LINEAR = 1 } gdr_rule;

typedef struct gdr_problem {
  int32_t B, T, H, HV, K, V; /* batch, tokens, q/k heads, value heads, key dim, value dim */
  int32_t chunk;             /* chunk length C: 32, 64 or 128, or 0 for the
                                automatic choice, which is 64 (faster than 32
                                and 128 on every workload measured);
                                negative: GDR_ERR_ARG */
  int32_t g_per_channel;     /* 0: g[B,T,HV]; 1: g[B,T,HV,K] */
  float scale;               /* query scale; callers usually pass 1/sqrt(K) */
  int32_t qkv_dtype;         /* gdr_dtype of q, k and v */
  int32_t scan_segments;     /* sequence segments of the state scan: 0 chooses
                                automatically (gdr_chunk_scan_segments), n > 0
                                asks for n (rounded so that every segment holds
                                the same number of chunks, at most one per chunk) */
  int32_t scan_slab;         /* state columns per state-scan workgroup: 0 chooses
                                automatically (gdr_chunk_scan_slab), or 32 or 64
                                (with 128-row chunks only 32 for K = 128 and 64
                                for K = 64 are built); any width gives the same
                                result up to rounding order, it only moves work
                                between workgroups */
  int32_t qk_l2norm;         /* 1: L2-normalise every q and k row inside the
                                kernels first, x * rsqrt(sum(x^2) + 1e-6) (the
                                scalar-g kernel page's optional normaliser);
                                the sums run in fp32 and each row's factor
                                multiplies its raw values in fp32 wherever
                                they enter a product.  0: q and k are used as
                                given */
  int32_t rule;              /* gdr_rule: GDR_RULE_DELTA (0) or GDR_RULE_LINEAR */
  int32_t o_dtype;           /* gdr_dtype of o: GDR_F32 (0, the default),
                                GDR_BF16 or GDR_F16, the fp32 result rounded
                                once to nearest even as it is stored (the
                                scalar-g kernel page casts its output back
                                to the input dtype).  Rounding o alone to
                                bf16 costs about 2e-2 relative to max|o| /
                                rms(o) on the workloads, so fp32 is the form
                                whose accuracy the library states. */
} gdr_problem;

/* Bytes of device workspace gdr_chunk_fwd needs for problem `p`, or 0 when
 * `p` is NULL or fails validation.  The size grows linearly with
 * B * HV * ceil(T / chunk). */
size_t gdr_chunk_fwd_workspace_size(const gdr_problem* p);

/* The whole forward pass: chunk preparation (cumsum, decayed dots, masks and
 * the UT inverse, all per chunk in parallel) followed by the state scan over
 * chunks.  Writes o for t < T and, when final_state is not NULL, the state
 * after token T-1.  T need not be a multiple of the chunk length: rows past T
 * are treated as padding with g = 0 and beta = 0, which leaves the state
 * unchanged. */
gdr_status gdr_chunk_fwd(const gdr_problem* p,
                         const void* q, const void* k, const void* v,
                         const float* g, const float* beta,
                         const float* initial_state,
                         void* o, float* final_state,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* gdr_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The workspace is the library's own
 * file-scope device array of GDR_NOALLOC_SCRATCH_BYTES (64 MiB) on the
 * current device; a problem whose gdr_chunk_fwd_workspace_size exceeds it
 * returns GDR_ERR_SCRATCH before anything is launched (the 4096-token,
 * 12-head, K = V = 128 problem needs about 49 MiB).  The caller still owns q,
 * k, v, g, beta, the states and o, with the layouts, validation, errors and
 * stream semantics of gdr_chunk_fwd; results equal gdr_chunk_fwd's bit for
 * bit.  No call here allocates or frees memory: the array's device address
 * is looked up once per device on that device's first call.  Every call on
 * one GPU shares that GPU's array, so calls that overlap in time on one GPU
 * (other streams, other host threads) race and must be serialised by the
 * caller.  Nothing in the array needs clearing between calls: each call
 * writes every byte it reads. */
gdr_status gdr_chunk_fwd_noalloc(const gdr_problem* p,
                                 const void* q, const void* k, const void* v,
                                 const float* g, const float* beta,
                                 const float* initial_state,
                                 void* o, float* final_state,
                                 void* stream);

/* Stage 1 alone (sec-03 notes: in-chunk cumsum, decayed dot, triangular
 * system; UT transform): fills the workspace for gdr_chunk_scan.  With the
 * inspection pointers non-NULL it also writes, in fp32 on the padded chunk
 * grid with N = ceil(T / chunk):
 *   gamma  [B, HV, N, C] (or [B, HV, N, C, K] per channel): in-chunk cumsum of g
 *   a_kk   [B, HV, N, C, C]: strictly lower A_kk with beta on columns (= M - I)
 *   a_qk   [B, HV, N, C, C]: lower A_qk (diagonal kept) with beta and scale
 *   m_inv  [B, HV, N, C, C]: M^-1, the UT transform's inverse
 * Any of them may be NULL. */
gdr_status gdr_chunk_prep(const gdr_problem* p,
                          const void* q, const void* k,
                          const float* g, const float* beta,
                          void* workspace, size_t workspace_bytes,
                          float* gamma, float* a_kk, float* a_qk, float* m_inv,
                          void* stream);

/* Stage 2 alone (sec-03 notes, inter-chunk recurrence): the scan over
 * chunks using a workspace filled by gdr_chunk_prep for the same problem and
 * the same q, k, g, beta.  r = U - W S, o = (q exp(gamma)) S + A_qk r,
 * S <- diag(exp(gamma_last)) S + (exp(gamma_last - gamma) k)^T (beta r),
 * with W = M^-1 (exp(gamma) k) and U = M^-1 v folded into the workspace.
 * When the problem has few independent (batch, value head) scans relative to
 * its length, the sequence is cut into segments: the state update is affine
 * in S, so each segment's transition and zero-start end state are computed
 * in parallel, combined serially, and the segments then rerun from their
 * true start states.  Those segment states are written into the workspace,
 * which this stage therefore also writes. */
gdr_status gdr_chunk_scan(const gdr_problem* p,
                          const void* q, const void* k, const void* v,
                          const float* initial_state,
                          void* o, float* final_state,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/* One decode step (the recurrent form of the same rule, for serving one
 * token at a time): for every batch b and value head hv, with
 * d = exp(g) (one value, or one per key channel when g_per_channel = 1),
 *     u  = v - (diag(d) S)^T k
 *     S' = diag(d) S + beta k u^T
 *     o  = scale S'^T q
 * (sec-03 notes: the naive recurrence the chunkwise form equals; "Chunkwise
 * parallel algorithms" page, section 2.1: the delta rule).  The problem
 * takes T = 1 (GDR_ERR_SHAPE otherwise); chunk and scan_segments are
 * ignored, and scan_slab sets the state columns per workgroup (0 chooses,
 * or 32, 64 or 128; capped at V; any other value is GDR_ERR_ARG): each
 * column's update depends on its own K entries only, so the width only
 * spreads one state over more or fewer workgroups.  Layouts are those of gdr_chunk_fwd with the token axis of
 * extent 1:
 *   q, k  [B, H, K]  qkv_dtype        v  [B, HV, V]  qkv_dtype
 *   g     [B, HV] or [B, HV, K] fp32  beta [B, HV]   fp32
 *   state_in  [B, HV, K, V] fp32, or NULL for a zero state
 *   state_out [B, HV, K, V] fp32 (required); state_out == state_in updates
 *             the state in place (a partial overlap is GDR_ERR_ALIAS)
 *   o     [B, HV, V] o_dtype (fp32, bf16 or fp16)
 * No workspace.  Validation, errors and streams as for gdr_chunk_fwd.  The
 * kernel reads and writes the state once: it is bound by HBM bandwidth. */
gdr_status gdr_decode_step(const gdr_problem* p,
                           const void* q, const void* k, const void* v,
                           const float* g, const float* beta,
                           const float* state_in, float* state_out, void* o,
                           void* stream);

/* Bits of the word gdr_check_inputs writes. */
typedef enum gdr_check_bit {
  GDR_CHECK_NONFINITE = 1,   /* a NaN or an infinity in q, k, v, g or beta
                                (in the encoding of their dtype) */
  GDR_CHECK_FP16_RANGE = 2,  /* bf16 q, k or v with |x| >= 65520, which rounds to
                                infinity in fp16 (q and k are exempt with
                                qk_l2norm = 1: they are scaled in fp32 first) */
  GDR_CHECK_DECAY_RANGE = 4  /* 16-bit inputs: within some chunk of the problem's
                                chunk length, the positive g of one channel (or
                                of the row decay) sum to more than 8 */
} gdr_check_bit;

/* Checks the inputs of gdr_chunk_fwd (or of the stage calls) for problem `p`
 * against the numeric preconditions of the numerics notes above, on the
 * device: one pass over q, k, v, g and beta, which are only read.  Sets
 * *flags (device memory, 4-byte aligned, not overlapping any input) to the
 * OR of the gdr_check_bit values of every violation found, 0 when there is
 * none; the word is written on `stream`, so read it after synchronising.
 * With GDR_F32 inputs only GDR_CHECK_NONFINITE can be set (every product is
 * fp32).  Validation (GDR_ERR_NULL, _SHAPE, _DTYPE, _ARG, _UNSUPPORTED,
 * _ALIGN, _ALIAS, _DEVICE) as for gdr_chunk_fwd; the state's own range
 * (see above) depends on the whole recurrence and is not checked.  The
 * pass is bound by HBM bandwidth on the inputs' bytes: an optional
 * validation step, not part of the forward pass. */
gdr_status gdr_check_inputs(const gdr_problem* p,
                            const void* q, const void* k, const void* v,
                            const float* g, const float* beta,
                            uint32_t* flags, void* stream);

/* Number of sequence segments the state scan of problem `p` uses (1: one
 * serial scan over all chunks), or 0 when `p` fails validation.  The
 * automatic choice comes from a cost model of the MI355X (256 compute
 * units) and the problem sizes only. */
int gdr_chunk_scan_segments(const gdr_problem* p);

/* State columns per state-scan workgroup for problem `p` (32 or 64), or 0
 * when `p` fails validation.  Narrow slabs spread each scan over more
 * workgroups, which shortens the serial chunk step when few scans run; wide
 * slabs read each chunk's operands fewer times.  The automatic choice uses
 * the problem sizes only. */
int gdr_chunk_scan_slab(const gdr_problem* p);

/* Static, never-NULL text for any status value (unknown values included). */
const char* gdr_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
