/*
 * hla.h -- C ABI of the MI355X (gfx950) forward path of second-order
 * Higher-order Linear Attention (HLA-2) and of the asymmetric AHLA operator.
 *
 * Defining passages ("Resumen Tecnico: Atencion Lineal de Orden Superior
 * (HLA)", gist.science/es/paper/2510.27258):
 *   section "1. HLA de Segundo Orden"  -- prefix moments, cross-summaries, the
 *       output q^T (S^K C^QV - G) and the ratio-normalised form;
 *   section "2. ... (AHLA)"           -- the asymmetric operator Q (K^T Q)(K^T V);
 *   section "4. Entrenamiento Paralelo mediante Escaneos Asociativos" --
 *       chunk-parallel evaluation by an exclusive Blelloch scan of segment
 *       summaries under a semidirect-product combine;
 *   section "Contribuciones Clave", item 2 -- masked operators with
 *       exponential decay;
 *   section "Resultados y Afirmaciones" -- O(d^2 + d dv) per-token streaming
 *       cost, strict causality (output t depends on tokens j <= t only).
 *
 * Operators computed (A = Q K^T, L = tril(A) with the diagonal):
 *   HLA_HLA2        o = tril(L L^T) V, i.e.
 *                   o_t = sum_{j<=t} sum_{i<=j} g^((t-i)+(t-j)) A[t,i] A[j,i] v_j
 *   HLA_HLA2_RATIO  the HLA_HLA2 numerator divided, row by row, by the same
 *                   double sum with v == 1 (no epsilon; a zero denominator
 *                   gives IEEE inf/NaN in that row)
 *   HLA_AHLA        o = (L L) V,  o_t = sum_{i<=t} sum_{j<=i} g^(t-j) A[t,i] A[i,j] v_j
 *   HLA_AHLA_RATIO  the AHLA numerator over the same sum with v == 1
 *   HLA_HLA3        third order (section "3. HLA de Tercer Orden": the product
 *                   A A^T A made strictly causal), read as o = tril(L L^T) L V:
 *                   o_t = sum_{m<=t} sum_{i<=m} sum_{j<=m}
 *                         g^((t-i)+(t-m)+(t-j)) A[t,i] A[m,i] A[m,j] v_j.
 *                   Without a decay: the second-order operator on the values
 *                   Y = L V (one chunked first-order pass into the workspace,
 *                   then the three second-order stages).  With a decay: three
 *                   chained first-order passes, Y = LA_g(Q, K, V),
 *                   Z = LA_g(Q, K, K), o = LA_{g^3}(Q, Z, Y), all in stage 3
 *   HLA_HLA3_RATIO  the HLA_HLA3 numerator over the same sum with v == 1: the
 *                   chain above and its twin on unit values, in fp32 (bf16
 *                   inputs on widened copies), divided row by row
 * g is the per-head decay (1 when gamma is NULL).  Decay reading ("Contribuciones
 * Clave", item 2, names masked operators with and without exponential decay):
 * every streaming summary of the variant decays by g per token, hence the
 * weights g^((t-i)+(t-j)) for HLA-2 and g^(t-j) for AHLA.  No 1/sqrt(d) or
 * other scaling is applied inside.
 *
 * Layout (all row-major, contiguous, device memory):
 *   q, k : [B][H][n][d]     v, o : [B][H][n][dv]    element type = dtype
 *   state: fp32, one block per (b,h) of hla_state_floats() floats:
 *     HLA-2 : [ S (d*d) | W (d*dv) | u (d) ]    S = sum g^(t-i) k_i k_i^T,
 *             W = S^K C^QV - G, u = S^K m^Q - h  (the page's five summaries
 *             folded into the three that a continuation needs)
 *     AHLA  : [ P (d*dv) | E (d*dv) | mK (d) | nk (d) ]  the page's P^KV, E, m^K, n
 *     HLA3  : not per (b,h) blocks: first the P^KV (d*dv) of every (b,h), then
 *             every (b,h)'s HLA-2 block [ S | W | u ] of (q, k, y), y = P^T q
 *             (hla_state_floats() = d*dv + d*d + d*dv + d per (b,h)); with a
 *             decay W = sum g^(3(t-m)) z_m y_m^T, and u is unused (written 0)
 *     HLA3_RATIO: the HLA3 layout twice: the chain on v, then the chain on
 *             unit values (1, 0, ..., 0) (hla_state_floats() = 2 x HLA3's)
 *
 * Ownership: the caller allocates and owns every buffer, including the
 * workspace.  The library allocates no memory, keeps no mutable global state,
 * never prints and never aborts.  All work is enqueued on `stream` (a
 * hipStream_t passed as void*, NULL = the null stream); the call returns
 * after enqueueing.  Concurrent calls on different streams are safe if they
 * use different workspaces and outputs.  Every device buffer must start on
 * a 16-byte boundary (the kernels move rows in 16-byte pieces; allocations
 * from hipMalloc or torch are 256-byte aligned); this is not checked.
 *
 * Errors: arguments are validated first, on the host, with no HIP call; on a
 * validation error nothing is enqueued.  A failed launch returns
 * HLA_ERR_DEVICE.  Faults inside kernels surface at the caller's next
 * synchronisation, as usual for HIP.
 */
#ifndef HLA_H
#define HLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HLA_OK = 0,
    HLA_ERR_NULL = 1,         /* a required pointer is NULL                     */
    HLA_ERR_SHAPE = 2,        /* B, H, d or dv < 1, or n < 0                     */
    HLA_ERR_UNSUPPORTED = 3,  /* no kernel for this (dtype, d, dv, chunk, variant) */
    HLA_ERR_WORKSPACE = 4,    /* workspace smaller than hla_workspace_bytes()    */
    HLA_ERR_DEVICE = 5,       /* a HIP launch or runtime call failed             */
    HLA_ERR_ARG = 6           /* bad enum value, gamma outside (0, 1], chunk or
                                 seg_chunks < 0                                  */
} hla_status;

typedef enum { HLA_F32 = 0, HLA_BF16 = 1 } hla_dtype;

typedef enum {
    HLA_HLA2 = 0,
    HLA_HLA2_RATIO = 1,
    HLA_AHLA = 2,
    HLA_AHLA_RATIO = 3,
    HLA_HLA3 = 4,
    HLA_HLA3_RATIO = 5
} hla_variant;

/* Largest H for which a per-head decay can be given (it travels in the kernel
 * arguments). */
#define HLA_MAX_DECAY_HEADS 256

/* Floats of streaming state per (b,h) for `variant` (see Layout above);
 * 0 for an unknown variant. */
size_t hla_state_floats(int variant, int d, int dv);

/* Segment length, in chunks, that hla_forward uses when seg_chunks == 0 (d is
 * the q/k head dimension: the segment summaries and the scan's combines grow
 * as d^2 dv, so at d >= 128 the default keeps half as many segments). */
int hla_default_seg_chunks(int variant, int B, int H, int n, int d, int chunk);

/* Bytes of device workspace hla_forward needs for these arguments
 * (seg_chunks == 0 means the default): 2*B*H*(nseg-1) fp32 summaries of
 * d*d + 2*d*dv + 2*d floats (the segment summaries and the nodes of the
 * scan's up-sweep).  0 when the sequence is one segment.  HLA_HLA3 adds
 * B*H*n*dv fp32 for Y and the segment states of its first-order pass. */
size_t hla_workspace_bytes(int variant, int B, int H, int n, int d, int dv,
                           int chunk, int seg_chunks);

/*
 * Chunked forward pass over a whole sequence.
 *
 * q, k, v, o     device pointers, layout above (may be NULL only if n == 0)
 * B, H, n, d, dv sizes; n may be any value >= 0 (a partial last chunk and a
 *                partial last segment are masked)
 * dtype          HLA_F32 (fp32 inputs, fp32 arithmetic and MFMA) or HLA_BF16
 *                (bf16 inputs and output, bf16 MFMA operands, fp32
 *                accumulation and fp32 state)
 * variant        hla_variant
 * gamma_host     NULL (no decay) or host array of H floats in (0, 1]: decay of
 *                head h, shared by every batch index; HLA-2 and AHLA
 *                variants (not HLA_HLA3), H <= HLA_MAX_DECAY_HEADS
 * chunk          tokens per intra-chunk tile: 16, 32 or 64 (see Supported)
 * seg_chunks     chunks per segment of the scan; 0 = hla_default_seg_chunks().
 *                The sequence is split into ceil(n / (chunk*seg_chunks))
 *                segments: their summaries are built in parallel, combined by
 *                an exclusive Blelloch scan (each segment forms its own
 *                exclusive prefix from the up-sweep nodes), and each
 *                segment's outputs are then computed from its carried state.
 * state_in       NULL (zero state) or device fp32 [B*H][hla_state_floats()]:
 *                the state after some earlier tokens; the pass continues it
 * state_out      NULL or device fp32 [B*H][hla_state_floats()]: receives the
 *                state after token n-1 (may not alias state_in)
 * workspace      device buffer of at least hla_workspace_bytes() bytes
 *                (may be NULL when that is 0); its contents on entry are
 *                ignored and on return are unspecified
 * stream         hipStream_t as void*
 *
 * Supported (otherwise HLA_ERR_UNSUPPORTED): d == dv, chunk 16, 32 or 64;
 *   HLA_BF16: d in {16, 32, 64, 128};
 *   HLA_F32:  d in {16, 32, 64};
 *   B*H <= 65535, and nseg*B*H <= 2^30 - 1, or 2^29 - 1 at dv >= 128
 *   (nseg = ceil(n / (chunk*seg_chunks)),
 *   one workgroup per segment and head).
 */
hla_status hla_forward(const void *q, const void *k, const void *v, void *o,
                       int B, int H, int n, int d, int dv, int dtype, int variant,
                       const float *gamma_host, int chunk, int seg_chunks,
                       const float *state_in, float *state_out,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * hla_forward that also writes, for every token, the rows of the first of
 * the operator's two chained passes, for a later hla_backward_z (which would
 * otherwise recompute them):
 *   HLA-2 forms: the keyed queries z_t = S^K_t q_t, S^K_t = sum_{s<=t}
 *     g^(t-s) k_s k_s^T (page section "1. HLA de Segundo Orden": the query
 *     keyed by the running key moment; Z = LA_g(Q, K, K)), rows of d;
 *   AHLA forms: y_t = P_t^T q_t, P_t = sum_{s<=t} g^(t-s) k_s v_s^T (section
 *     "2. ... (AHLA)": the first-order pass; Y = LA_g(Q, K, V)), rows of dv.
 *
 * z   device, [B][H][n][d] (HLA-2) or [B][H][n][dv] (AHLA), element type =
 *     dtype; not q, k, v or o.  Each row is rounded once from its fp32
 *     accumulation, as the forward stages it for its own products.
 * Other arguments, results and errors as hla_forward (o is bit for bit the
 * same).  variant: HLA_HLA2, HLA_HLA2_RATIO, HLA_AHLA or HLA_AHLA_RATIO (z
 * does not depend on the ratio), otherwise HLA_ERR_UNSUPPORTED; z NULL with
 * n > 0: HLA_ERR_NULL; z equal to q, k, v or o: HLA_ERR_ARG.
 */
hla_status hla_forward_z(const void *q, const void *k, const void *v, void *o, void *z,
                         int B, int H, int n, int d, int dv, int dtype, int variant,
                         const float *gamma_host, int chunk, int seg_chunks,
                         const float *state_in, float *state_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The three stages hla_forward runs, one at a time, on the same arguments
 * (page section "4. ... Escaneos Asociativos": segment summaries combined by
 * an exclusive Blelloch scan under the semidirect-product combine).  With
 * SUMF = d*d + 2*d*dv + 2*d, R = nseg-1, parts X | Y | N | y | nv:
 *   stage 1  the summary of segment s, s = 0 .. R-1, into the leaf at floats
 *            ws + (bh*R + s)*SUMF;
 *   stage 2  the up-sweep of the scan: node (b, m), b >= 1, the combine of
 *            segments m*2^b .. (m+1)*2^b - 1, for every such node that ends
 *            below R, at ws + (B*H*R + bh*R + i)*SUMF, where i counts the
 *            nodes of levels 1 .. b-1 (R >> l of them at level l) plus m;
 *   stage 3  for every segment s, the initial state and the nodes that tile
 *            segments 0 .. s-1 (one per set bit of s) folded into its carried
 *            state (what the scan's down-sweep delivers), then the chunked
 *            forward from that state, and state_out.
 * With R <= 3 (at most four segments) the scan has no up-sweep: stage 2
 * enqueues nothing, the node slots stay unused, and stage 3 folds the leaves
 * 0 .. s-1 of segment s one by one (at most three folds cost less than the
 * up-sweep's launch).
 * Calling stages 1, 2, 3 in order on one stream with identical arguments is
 * exactly hla_forward.  With a single segment stages 1 and 2 enqueue nothing.
 * Meant for callers that time the stages or place them themselves (a caller
 * that shards a sequence can exchange segment summaries between stages 1 and
 * 2).  Returns HLA_ERR_ARG for a stage outside 1..3, otherwise as hla_forward.
 */
hla_status hla_forward_stage(int stage, const void *q, const void *k, const void *v, void *o,
                             int B, int H, int n, int d, int dv, int dtype, int variant,
                             const float *gamma_host, int chunk, int seg_chunks,
                             const float *state_in, float *state_out,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * hla_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as hla_forward, without the workspace
 * arguments: the workspace is a fixed array of HLA_NOALLOC_SCRATCH_BYTES
 * inside the library, one copy per device, held by each device the library
 * runs on until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocating library routine); the caller still passes q, k, v, o and the
 * states.  The first call on a device looks up the array's address there
 * (one hipGetSymbolAddress).
 *
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (nothing in it needs clearing: every part a call reads it
 * writes first).  Calls that overlap in time on one device -- on different
 * streams or from different threads without ordering -- race on the array and
 * give wrong results; calls on one stream are ordered and safe.
 *
 * Errors: as hla_forward, plus HLA_ERR_WORKSPACE when the call needs more
 * than HLA_NOALLOC_SCRATCH_BYTES of workspace (hla_workspace_bytes() with
 * the same arguments; a larger seg_chunks means fewer segments and a smaller
 * workspace), and HLA_ERR_DEVICE when the array's address cannot be found.
 * 64 MiB covers, e.g., B*H = 128, n = 4096, d = dv = 64 with the default
 * segments (38 MB).
 */
#define HLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hla_status hla_forward_noalloc(const void *q, const void *k, const void *v, void *o,
                               int B, int H, int n, int d, int dv, int dtype, int variant,
                               const float *gamma_host, int chunk, int seg_chunks,
                               const float *state_in, float *state_out, void *stream);

/*
 * One streaming (decode) step: for every (b,h) take the single token
 * q, k : [B][H][d], v : [B][H][dv], update `state` in place and write
 * o : [B][H][dv].  The update is the same recurrence the forward pass
 * carries between chunks (page section "1. HLA de Segundo Orden",
 * "Resultados y Afirmaciones": constant state, O(d^2 + d dv) per token):
 *   HLA-2: S <- g S + k k^T; z = S q; W <- g^2 W + z v^T; u <- g^2 u + z;
 *          o = q^T W  (ratio: / q^T u)
 *   AHLA : P <- P + k v^T; y = P^T q; E <- E + k y^T; mK <- mK + k;
 *          nk <- nk + k (q . mK); o = q^T E  (ratio: / q^T nk)
 *   HLA3 : P <- P + k v^T; y = P^T q; then the HLA-2 step on (q, k, y)
 * state is device fp32 [B*H][hla_state_floats()], never NULL.
 */
hla_status hla_step(const void *q, const void *k, const void *v, void *o,
                    int B, int H, int d, int dv, int dtype, int variant,
                    const float *gamma_host, float *state, void *stream);

/*
 * Backward pass (vector-Jacobian product) of the HLA-2 and AHLA operators,
 * for training through the chunk-parallel form (page section "4.
 * Entrenamiento Paralelo mediante Escaneos Asociativos"; the operators of
 * sections "1. HLA de Segundo Orden" and "2. ... (AHLA)", decay per
 * "Contribuciones Clave" item 2).  Given the upstream gradient dout = dL/do,
 * writes dq = dL/dq, dk = dL/dk, dv = dL/dv of the HLA_HLA2 output
 * o = tril(L L^T) V (with decay g_h when gamma_host is given), of the
 * HLA_AHLA output o = (L L) V, or of either ratio form (HLA_HLA2_RATIO,
 * HLA_AHLA_RATIO), computed from zero state.
 *
 * Method: with z_t = S^K_t q_t, the operator is two chained causal linear
 * attentions, Z = LA_g(Q, K, K) and O = LA_{g^2}(Q, Z, V), where
 * LA_g(A, B, C)_t = sum_{s<=t} g^(t-s) (a_t . b_s) c_s.  The chain rule through
 * each gives linear attentions of the same form, causal or anti-causal; the
 * library runs five chunked passes (chunk 64 tokens, segments of seg_chunks
 * chunks in parallel, each pass a segment-state launch and a main launch;
 * the last pass reuses the first one's segment states), recomputing Z, and
 * keeps Z and dZ in the workspace.  AHLA is LA(Q, K, LA(Q, K, V)): five
 * passes likewise, with Y = LA(Q, K, V) and dY in the workspace.  The ratio
 * form recomputes num and den (two more passes and a row-wise kernel), runs
 * the passes with dO / den as upstream gradient, and adds the denominator's
 * terms through one more pass; it keeps three more tensors in the workspace.
 * The AHLA ratio form runs the AHLA chain twice (upstream dO / den on V, and
 * the denominator's upstream on unit rows), with two more tensors.
 *
 * q, k, v, dout  device, [B][H][n][d] (d == dv), element type = dtype
 * dq, dk, dv_out  device outputs, same layout and type; may not alias the
 *                inputs or each other
 * gamma_host     NULL or H decays in (0, 1] (as hla_forward)
 * dgamma         NULL, or device [H] fp32 output (HLA_HLA2, HLA_HLA2_RATIO):
 *                dL/dg_h, summed over the batch, at the decays given (1 for
 *                every head when gamma_host is NULL).  Differentiating each
 *                g^(t-s) factor of the two chained passes gives
 *                g_h dL/dg_h = sum_{b,t} (t - c)(2 q_t.dq_t - 3 z_t.dz_t
 *                - k_t.dk_t / 2) for any constant c, with Z and dZ as kept
 *                in the workspace; two more launches form it (fp32 row terms
 *                summed in fp64 in a fixed order, so repeat calls agree
 *                bit for bit).  Those terms nearly cancel, so with dgamma
 *                every pass runs in fp32 (bf16 inputs on widened copies):
 *                bf16 intermediates would leave dL/dg a few percent off.
 *                n == 0 writes zeros.  Non-NULL with an AHLA form:
 *                HLA_ERR_UNSUPPORTED.
 * seg_chunks     chunks (of 64 tokens) per segment; 0 = the library's default
 *                (hla_backward_default_seg_chunks)
 * workspace      device buffer of at least hla_backward_workspace_bytes()
 *                bytes, with_dgamma = (dgamma != NULL) (contents ignored on
 *                entry, unspecified on return)
 * Precision: bf16 operands, fp32 accumulation and fp32 carried states; Z and
 * dZ are kept in dtype; the ratio forms, and every form when dgamma is
 * given, run every pass in fp32 (for bf16 inputs on widened copies).
 * Supported: every variant, with or without a decay (the ratio forms need
 * nonzero denominators, as the forward), d == dv in {16, 32, 64, 128}, both
 * dtypes.  With a decay, AHLA is LA_g(Q, K, LA_g(Q, K, V)) and its passes
 * carry g.  Third order is Y = LA_g(Q, K, V), Z = LA_g(Q, K, K),
 * O = LA_{g^3}(Q, Z, Y): its gradient is eight passes (the ratio form, run
 * in fp32, thirteen: the unit-value chain as well).  dgamma is for the HLA-2
 * forms only.  Errors as hla_forward.
 */
int hla_backward_default_seg_chunks(int B, int H, int n);
size_t hla_backward_workspace_bytes(int variant, int B, int H, int n, int d, int dv, int dtype,
                                    int seg_chunks, int with_dgamma);
hla_status hla_backward(const void *q, const void *k, const void *v, const void *dout,
                        void *dq, void *dk, void *dv_out, int B, int H, int n, int d, int dv,
                        int dtype, int variant, const float *gamma_host, float *dgamma,
                        int seg_chunks, void *workspace, size_t workspace_bytes, void *stream);

/*
 * hla_backward of the HLA_HLA2 or HLA_AHLA output (with or without a decay)
 * given the rows z that hla_forward_z wrote for the same q, k, v and decays.
 * HLA-2: the first pass's main launch, Z = LA_g(Q, K, K), is skipped (its
 * segment states of K K^T are still formed, for the last pass).  AHLA: the
 * first pass, Y = LA_g(Q, K, V), is skipped whole.  Four passes remain.
 *
 * z   device, [B][H][n][d], element type = dtype, as hla_forward_z wrote it;
 *     not dq, dk or dv_out.
 * Other arguments as hla_backward, without dgamma (the decay gradient's
 * passes run in fp32 and recompute Z; use hla_backward for it); the same
 * workspace size (hla_backward_workspace_bytes with with_dgamma = 0).
 * Results: those of hla_backward up to the rounding of Z (the forward's
 * row for row instead of the backward's own recomputation of it).
 * Errors as hla_backward; variant other than HLA_HLA2 or HLA_AHLA:
 * HLA_ERR_UNSUPPORTED;
 * z NULL with n > 0: HLA_ERR_NULL; z equal to an output: HLA_ERR_ARG.
 */
hla_status hla_backward_z(const void *q, const void *k, const void *v, const void *z,
                          const void *dout, void *dq, void *dk, void *dv_out, int B, int H,
                          int n, int d, int dv, int dtype, int variant, const float *gamma_host,
                          int seg_chunks, void *workspace, size_t workspace_bytes, void *stream);

/* Unmasked (non-causal) second-order operators: the operators of sections
 * "1. HLA de Segundo Orden" and "2. ... (AHLA)" without the causal masks,
 * i.e. the products of the moments over the whole sequence:
 *     variant HLA_HLA2:  o = (Q K^T)(K Q^T) V = Q (K^T K)(Q^T V)
 *     variant HLA_AHLA:  o = (Q K^T)(Q K^T) V = Q (K^T Q)(K^T V)
 * Every output row sees every token, so there is no streaming state, decay
 * or decode step.  Three launches on `stream`: per-block fp32 partial sums of
 * the two d x d moments, their sum (in a fixed order) and product T, then
 * o_t = T^T q_t.  fp32 inputs: fp32 arithmetic throughout.  bf16 inputs:
 * the moment sums on bf16 MFMA with fp32 accumulation, T in fp32, and for
 * d >= 32 the read-out on bf16 MFMA with T rounded to bf16.
 *
 * q, k, v, o  device, [B][H][n][d] (dv == d), element type = dtype
 * workspace   device buffer of at least hla_unmasked_workspace_bytes() bytes
 *             (B*H*(2*nblk + 1)*d*d fp32 and B*H*d*d bf16, nblk <= 64
 *             partial blocks per head)
 * Supported: HLA_HLA2 and HLA_AHLA only (the ratio forms and
 * HLA_HLA3: HLA_ERR_UNSUPPORTED), d in {16, 32, 64, 128} for both dtypes.
 * n == 0: nothing to do, HLA_OK.  Errors as hla_forward. */
size_t hla_unmasked_workspace_bytes(int B, int H, int n, int d);
hla_status hla_unmasked_forward(const void *q, const void *k, const void *v, void *o, int B,
                                int H, int n, int d, int dtype, int variant, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *hla_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* HLA_H */
