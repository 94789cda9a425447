/*
 * gdn2.h -- C ABI of libgdn2, the MI355X (gfx950) hot path (forward, backward
 * and decode) of the Gated DeltaNet-2 (GDN-2) sequence-mixing recurrence.
 *
 * The operation (one head; state S is dk x dv float32, row i = key channel,
 * column j = value channel).  For every token t, in order:
 *
 *   D   = Diag(alpha_t) S          per-key-channel decay, applied first
 *   z   = w_t (.) v_t - D^T (b_t (.) k_t)
 *   S   = D + k_t z^T
 *   o_t = S^T q_t                  (read after the update, no 1/sqrt(dk))
 *
 * Sources: the formal paragraph of the aixai.ru blog ("Gated DeltaNet-2",
 * section on why one scalar cannot serve both decisions: the decay is
 * applied first, b enters the read of the state, w gates the value
 * written); aiexpert.news/pt (method paragraph: b_t in
 * [0,1]^dk on the key axis, w_t in [0,1]^dv on the value axis, per-channel
 * decay kept from KDA, exact reduction to KDA when b and w collapse to one
 * scalar); aixai.ru, implementation section (chunkwise parallel form, q and k
 * L2-normalised outside the kernel).  The pages print no formula; the rule
 * above is the plainest reading that reduces to KDA, Gated DeltaNet and
 * DeltaNet exactly.  No gate is clamped: b in [0,2] is accepted (aixai.ru,
 * ablation section).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous,
 *     token-major: q, k, alpha, b are [B, T, H, dk]; v, w, o are [B, T, H, dv].
 *     With packed sequences (cu_seqlens != NULL) B must be 1 and T is the total
 *     token count.  States are [N, H, dk, dv] float32 (row-major dk x dv per
 *     head).  Pointers must be 16-byte aligned.
 *   - The element type of q, k, v, alpha, b, w and o is given by `dt`
 *     (float32 or bfloat16); arithmetic is float32 and states are float32.
 *     bfloat16 outputs are rounded to nearest even.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every kernel is enqueued on it; the library never synchronises it and
 *     allocates no memory.
 *   - Errors that the host can detect (null pointer, unsupported size or
 *     dtype, workspace too small, inconsistent sizes) are returned before any
 *     launch, with a message in gdn2_last_error().  A failed launch returns
 *     GDN2_ERR_HIP.  Conditions only the device could see (a non-monotone
 *     cu_seqlens, NaN/Inf inputs) are not detected: NaN propagates to the
 *     outputs of its sequence and head.
 *   - Supported sizes: dk and dv each in {16, 32, 64, 128}; chunk in
 *     {16, 64}.  gdn2_chunk_fwd, gdn2_chunk_bwd and gdn2_decode_step take
 *     dk != dv; the segment maps and their combine, and the allocation-free
 *     forward take dk == dv (GDN2_ERR_UNSUPPORTED otherwise).  The decode
 *     step and the token-by-token path are built for every (dk, dv) pair.
 *     The chunked paths run a call with dk != dv on d = max(dk, dv): the
 *     narrower side's inputs are widened in the front of the workspace with
 *     channels that cannot reach the result (extra key channels with
 *     q = k = b = 0 and no decay, whose state rows stay zero; extra value
 *     channels with v = w = 0, whose state columns stay zero), the d x d
 *     call runs, and o and S_final (the backward: the gradients and dS0)
 *     are narrowed back.
 *   - Decay range: any alpha in [0, 1], alpha = 0 (a full erase of that
 *     channel) included, on every path.  The chunked kernels build every
 *     decay factor from sums of log decays (never the difference of two
 *     prefix sums) and form the diagonal 16-token blocks pair by pair, from
 *     running products of the alphas, wherever a 16-token stretch decays by
 *     more than 2^-64 (the pages keep the log-decay in float32 because the
 *     in-chunk cumulative sum is precision-sensitive: aixai.ru blog, section
 *     on how the method is implemented in practice).  The backward's
 *     gradient with respect to alpha itself is d(ln alpha) / alpha: its
 *     error grows as 1 / alpha and alpha = 0 gives no finite value; the
 *     log-decay input (GDN2_FLAG_LAYER_PREP) returns d(ln alpha) directly
 *     for every decay.
 */
#ifndef GDN2_H
#define GDN2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN2_ABI_VERSION 1

/* The *_MAX_ENUM values are never returned or accepted: they give both
 * enums the range of a non-negative int, so that any such value a caller
 * passes (an unknown status or dtype) is a valid value of the type and is
 * refused by the library, not undefined. */
typedef enum {
    GDN2_OK = 0,
    GDN2_ERR_INVALID_ARGUMENT = 1,
    GDN2_ERR_UNSUPPORTED = 2,
    GDN2_ERR_WORKSPACE_TOO_SMALL = 3,
    GDN2_ERR_HIP = 4,
    GDN2_STATUS_MAX_ENUM = 0x7FFFFFFF
} gdn2_status_t;

typedef enum { GDN2_F32 = 0, GDN2_BF16 = 1, GDN2_DTYPE_MAX_ENUM = 0x7FFFFFFF } gdn2_dtype_t;

/* flags of gdn2_chunk_fwd */
#define GDN2_FLAG_RECURRENT (1u << 1) /* token-by-token kernel instead of the
                                         chunked kernels (cross-check path) */
#define GDN2_FLAG_TWO_PASS (1u << 2)  /* chunked path: force the two-pass kernels */
#define GDN2_FLAG_FUSED (1u << 3)     /* chunked path: force the single-pass kernel
                                         (GDN2_ERR_UNSUPPORTED where it has none:
                                         chunk 64 needs dk in {64, 128}, and
                                         float32 with dk = 128 needs chunk 16) */
/* Gate layout flags (chunked paths only; GDN2_ERR_UNSUPPORTED with
 * GDN2_FLAG_RECURRENT).  Each makes one input a single value per (token,
 * head), laid out [B, T, H] (packed: [1, T, H]) in dtype dt and shared by all
 * channels of that token and head.  b = w = beta with both gate flags is KDA
 * (aiexpert.news/pt, method paragraph: GDN-2 reduces exactly to KDA when both
 * gates collapse to one scalar); adding GDN2_FLAG_SCALAR_ALPHA gives Gated
 * DeltaNet (needhelp.icu/de, section on the generalisation hierarchy).  One
 * gate flag alone gives the single-gate ablations (aixai.ru blog, ablation
 * paragraph). */
#define GDN2_FLAG_SCALAR_B (1u << 4)     /* b is [B, T, H] */
#define GDN2_FLAG_SCALAR_W (1u << 5)     /* w is [B, T, H] */
#define GDN2_FLAG_SCALAR_ALPHA (1u << 6) /* alpha is [B, T, H] */
/* Layer prep (chunked paths only; GDN2_ERR_UNSUPPORTED with
 * GDN2_FLAG_RECURRENT).  The inputs are the layer's raw projections as the
 * aixai.ru blog describes them (section on how the method is implemented in
 * practice): q and k not yet L2-normalised, the gates b and w as logits
 * (the kernel applies the logistic sigmoid, giving the [0, 1] gates of
 * aiexpert.news/pt), and alpha as the float32 natural-log decay
 * g = ln(alpha) <= 0, computed outside the kernel: alpha then points to
 * float32 data whatever dt is ([B, T, H, dk], or [B, T, H] with
 * GDN2_FLAG_SCALAR_ALPHA).  The kernels L2-normalise q and k per (token,
 * head) in float32 (a zero row stays zero). */
#define GDN2_FLAG_LAYER_PREP (1u << 0)
/* Rule R1.  The alternative reading of the pages' formal paragraph
 * (aixai.ru blog, gate section) in which the erase gate places the erased
 * direction instead of weighting the read:
 *   D = Diag(alpha) S;  r = D^T k;  S = D - (b (.) k) r^T + k (w (.) v)^T;
 *   o = S^T q.
 * It reduces to KDA, Gated DeltaNet and DeltaNet as the default rule does;
 * the pages do not settle which of the two they mean.  It runs on the
 * token-by-token path (with GDN2_FLAG_RECURRENT) and on the chunked two-pass
 * path (the default path or GDN2_FLAG_TWO_PASS; never the segment schedule),
 * with any gate layout and layer prep; with GDN2_FLAG_FUSED or
 * GDN2_FLAG_PREPARED it returns GDN2_ERR_UNSUPPORTED, and so it does for
 * float32 with dk = 128 and chunk 64.  Its chunked path needs the workspace
 * gdn2_chunk_fwd_workspace_bytes_flags reports for this flag (larger
 * per-chunk blocks). */
#define GDN2_FLAG_RULE_R1 (1u << 7)
/* Prepared workspace (two-pass path only; GDN2_ERR_UNSUPPORTED with
 * GDN2_FLAG_RECURRENT or GDN2_FLAG_FUSED).  For the caller that has just run
 * gdn2_chunk_segment_map on the same inputs, sizes, gate flags and workspace:
 * a context-parallel rank that computes its segment's map, exchanges the
 * maps, and then runs its segment from the true entering state.  The
 * workspace already holds every chunk's intermediates (they do not depend
 * on S0), so gdn2_chunk_fwd skips the per-chunk kernel and runs the state
 * scan alone; q .. w are checked but not read.  A workspace filled by
 * gdn2_chunk_fwd on the two-pass path serves the same way.
 * gdn2_chunk_bwd takes it too (dk == dv only): a training step that has
 * run gdn2_chunk_fwd with GDN2_FLAG_TWO_PASS on the same inputs, sizes and
 * gate flags, into the front of the backward's own workspace (at least
 * gdn2_chunk_bwd_workspace_bytes), hands those intermediates to the
 * backward, which then skips its own per-chunk kernel (it still reads
 * q .. w for the gradients).  The results are those of the backward without
 * the flag, bit for bit.  Any other contents give undefined outputs. */
#define GDN2_FLAG_PREPARED (1u << 8)
/* Kept states, for a training step (dk == dv, two-pass path only; implies
 * GDN2_FLAG_TWO_PASS; GDN2_ERR_UNSUPPORTED with GDN2_FLAG_RECURRENT,
 * GDN2_FLAG_FUSED, GDN2_FLAG_RULE_R1 or dk != dv).  gdn2_chunk_fwd's state
 * scan then also writes the state entering every chunk (the state the
 * chunked recurrence carries between chunks: aixai.ru blog, section on how
 * it is implemented in practice) into the workspace, where the backward
 * keeps its states; the workspace must then hold at least
 * gdn2_chunk_fwd_workspace_bytes_flags(..., flags) bytes (the backward's
 * size), and the segment schedule is not taken.  gdn2_chunk_bwd takes the
 * flag together with GDN2_FLAG_PREPARED (GDN2_ERR_UNSUPPORTED alone): the
 * workspace holds the blocks and states of such a forward on the same
 * inputs, S0, sizes and gate flags, and the backward skips its states scan
 * too.  For shapes where the backward takes the segment schedule it still
 * computes the segment maps (for the state gradients) but not the states;
 * there the kept states (one scan) differ from the segment schedule's in
 * rounding only.  At every other shape the gradients are those of the
 * backward without the flags, bit for bit. */
#define GDN2_FLAG_KEEP_STATES (1u << 9)

/* Size limits of every chunked entry point (gdn2_chunk_fwd, its
 * allocation-free variant, gdn2_chunk_bwd, gdn2_chunk_segment_map): at most
 * 2^40 input elements (B T H dk), fewer than 2^24 chunk-heads (chunk slots
 * x H: one workgroup each, whose work-items a dispatch counts in 32 bits),
 * at most 2^21 sequence-heads (sequences x H).  Larger calls return
 * GDN2_ERR_UNSUPPORTED before any launch, and the workspace-size functions
 * return 0 for them.  gdn2_decode_step takes fewer than 2^24
 * sequence-heads. */

/* Bytes of device workspace gdn2_chunk_fwd needs for these sizes (0 when
 * the sizes are unsupported).  With cu_seqlens, pass the packed total T and
 * the sequence count num_seqs; without, num_seqs is ignored (it is B).  For
 * a few long sequences the figure includes the segment schedule's maps (see
 * gdn2_chunk_fwd, flags). */
size_t gdn2_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs,
                                      int chunk, gdn2_dtype_t dt);

/* The same for a given set of gdn2_chunk_fwd flags: with GDN2_FLAG_RULE_R1
 * on the chunked path the per-chunk blocks are larger; with
 * GDN2_FLAG_KEEP_STATES it is gdn2_chunk_bwd_workspace_bytes (0 when
 * dk != dv); for every other set of flags it equals
 * gdn2_chunk_fwd_workspace_bytes. */
size_t gdn2_chunk_fwd_workspace_bytes_flags(int B, int T, int H, int dk, int dv, int num_seqs,
                                            int chunk, gdn2_dtype_t dt, uint32_t flags);

/* Chunkwise-parallel forward over whole sequences (aixai.ru blog, section on
 * how it is implemented in practice: chunks with matrix products inside,
 * in-chunk auxiliary WY matrices; aiexpert.news/pt: chunkwise WY algorithm
 * with the decay absorbed into the erase factors).
 *   q, k, v, alpha, b, w : inputs (see conventions).
 *   S0        : initial states [N, H, dk, dv] float32, or NULL for zeros.
 *   cu_seqlens: device int32 [N + 1] with cu_seqlens[0] = 0 and
 *               cu_seqlens[N] = T (packed sequences, B = 1), or NULL for B
 *               sequences of length T (then N = B).  Chunks restart at every
 *               sequence boundary.
 *   B, T, H, dk, dv, num_seqs, chunk, dt : sizes; chunk is the chunk length.
 *   flags     : at most one of GDN2_FLAG_RECURRENT, GDN2_FLAG_TWO_PASS,
 *               GDN2_FLAG_FUSED, plus any of the gate layout flags,
 *               GDN2_FLAG_PREPARED and GDN2_FLAG_KEEP_STATES (both imply
 *               the two-pass path).  With no
 *               path flag the library runs the two-pass chunked kernels (all
 *               chunks in parallel, then the state scan).  For N
 *               sequences (B, or num_seqs packed) of at least 128 chunks (on
 *               average, packed) with N H <= 32, given the workspace
 *               gdn2_chunk_fwd_workspace_bytes reports for them, the default
 *               path cuts every sequence into G = min(16, 128 / (N H),
 *               chunks / 16) segments of whole chunks (4, 8 or 16; bounds
 *               computed on the device from cu_seqlens when packed): the
 *               segments' state maps (as gdn2_chunk_segment_map; none for a
 *               sequence's last segment), their scan from S0 (as
 *               gdn2_segment_combine), and every segment's state scan from
 *               its entering state (the last one's gives S_final), so
 *               that more compute units share the sequential scan; with a
 *               smaller workspace it runs the plain two-pass kernels.
 *               GDN2_FLAG_FUSED
 *               runs the single-pass kernel (one workgroup per head walks its
 *               chunks, no workspace traffic).  All choices compute the same
 *               recurrence.
 *   o         : output [B, T, H, dv], element type dt.
 *   S_final   : final states [N, H, dk, dv] float32, or NULL.  May alias S0.
 *   workspace : device scratch of at least
 *               gdn2_chunk_fwd_workspace_bytes(...) bytes (NULL allowed when
 *               that is 0).  Its contents on entry are irrelevant, except
 *               with GDN2_FLAG_PREPARED.  On return (two-pass path) it holds
 *               the chunks' intermediates (with dk != dv: after the widened
 *               copies of the inputs and one d x d state per sequence-head).
 * T == 0 is allowed: nothing but S_final = S0 (or zeros) is written. */
gdn2_status_t gdn2_chunk_fwd(const void *q, const void *k, const void *v, const void *alpha,
                             const void *b, const void *w, const float *S0,
                             const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                             int num_seqs, int chunk, gdn2_dtype_t dt, uint32_t flags, void *o,
                             float *S_final, void *workspace, size_t workspace_bytes,
                             void *stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): gdn2_chunk_fwd on the two-pass kernels without a workspace
 * argument.  The per-chunk intermediates go to a scratch array the library
 * holds in device memory, GDN2_NOALLOC_SCRATCH_BYTES on every GPU it runs
 * on, kept until the process ends; no memory is allocated per call.
 *   Arguments: as gdn2_chunk_fwd, minus the workspace.  flags: the gate
 *   layout and layer prep flags (GDN2_FLAG_TWO_PASS is accepted and
 *   implied); the path, rule and prepared-workspace flags return
 *   GDN2_ERR_UNSUPPORTED.
 *   Sizes: a call whose two-pass workspace (gdn2_chunk_fwd_workspace_bytes
 *   without the segment schedule) fits the scratch runs as one
 *   gdn2_chunk_fwd call.  A larger fixed-length call (cu_seqlens == NULL)
 *   runs every sequence in pieces of whole chunks, in order, each piece
 *   starting from the state the previous one left (kept in S_final, or in
 *   the scratch when S_final is NULL); the results equal gdn2_chunk_fwd's
 *   on the two-pass path exactly.  Larger packed input, one chunk of H heads
 *   that does not fit, or pieces that would misalign a per-(token, head)
 *   gate tensor return GDN2_ERR_WORKSPACE_TOO_SMALL or GDN2_ERR_UNSUPPORTED
 *   before any launch.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (several host threads, or several streams without
 *   ordering between them) race and give undefined outputs.  Nothing in the
 *   scratch needs to start at zero. */
#define GDN2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn2_status_t gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *alpha,
                                     const void *b, const void *w, const float *S0,
                                     const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                                     int num_seqs, int chunk, gdn2_dtype_t dt, uint32_t flags, void *o,
                                     float *S_final, void *stream);

/* Bytes of device workspace gdn2_chunk_bwd needs for these sizes (0 when
 * the sizes are unsupported); num_seqs as for gdn2_chunk_fwd_workspace_bytes.
 * For a few long sequences the figure includes the segment schedule's maps
 * (see gdn2_chunk_bwd). */
size_t gdn2_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs,
                                      int chunk, gdn2_dtype_t dt);

/* Chunked backward: the gradients of a scalar loss L through the forward
 * above (the same recurrence, inputs and sizes as gdn2_chunk_fwd), with both
 * gates differentiated inside the chunked products (aiexpert.news/pt, method
 * paragraph: the gate-aware backward; aixai.ru blog, section on how the
 * method is implemented in practice).
 *   q .. cu_seqlens, B .. dt : the forward's inputs and sizes.
 *   flags     : GDN2_FLAG_SCALAR_B / _W / _ALPHA and GDN2_FLAG_LAYER_PREP,
 *               with the forward's meaning (inputs given per (token, head),
 *               or the raw layer inputs), GDN2_FLAG_PREPARED (the
 *               workspace's front holds the forward's per-chunk blocks, see
 *               that flag; GDN2_ERR_UNSUPPORTED when dk != dv) and, with it,
 *               GDN2_FLAG_KEEP_STATES (the workspace also holds the
 *               forward's kept states); the path and rule flags return
 *               GDN2_ERR_UNSUPPORTED.
 *   dout      : dL/do [B, T, H, dv], element type dt.
 *   dS_final  : dL/dS_final [N, H, dk, dv] float32, or NULL for zero.
 *   dq, dk_out, dv_out, dalpha, db, dw : outputs, the gradients with respect
 *               to the inputs as given: each has its input's layout and
 *               element type (dt; under layer prep dalpha is float32 like
 *               the log-decay input), bfloat16 rounded to nearest even.
 *               Without layer prep dalpha is the gradient with respect to
 *               alpha itself; with it, with respect to ln(alpha), and dq,
 *               dk, db, dw are taken through the L2 normalisation and the
 *               sigmoids (a zero q or k row gets a zero gradient).  An input
 *               given per (token, head) gets the sum of its channels'
 *               gradients.
 *   dS0       : dL/dS0 [N, H, dk, dv] float32, or NULL.
 *   workspace : device scratch of at least gdn2_chunk_bwd_workspace_bytes(...)
 *               bytes; its contents on entry are irrelevant without
 *               GDN2_FLAG_PREPARED (with dk != dv its front holds the
 *               widened inputs, dout, their gradients and three d x d states
 *               per sequence-head).
 * The kernels recompute the forward's per-chunk quantities (unless
 * GDN2_FLAG_PREPARED hands them over) and the state entering every chunk; no
 * forward output needs to be kept.  For the shapes
 * where gdn2_chunk_fwd takes its segment schedule (a few long sequences),
 * given the workspace gdn2_chunk_bwd_workspace_bytes reports, both of the
 * backward's scans take it too: the states from the segment maps and their
 * scan, the state gradients from per-segment reverse scans and the adjoint
 * scan of the maps (Phi transposed, from the last segment).  Decay range:
 * see the conventions above (dalpha with respect to alpha itself needs
 * alpha > 0; under layer prep every decay, -inf log included, works). */
gdn2_status_t gdn2_chunk_bwd(const void *q, const void *k, const void *v, const void *alpha,
                             const void *b, const void *w, const float *S0,
                             const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                             int num_seqs, int chunk, gdn2_dtype_t dt, uint32_t flags,
                             const void *dout, const float *dS_final, void *dq, void *dk_out,
                             void *dv_out, void *dalpha, void *db, void *dw, float *dS0,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Affine state map of sequence segments (context parallelism along T: a
 * long sequence cut into segments that run side by side).  Over any run of
 * tokens the recurrence above is affine in the state it starts from,
 *   S_out = Phi S_in + Psi,
 * because every token's update is (Diag(alpha) - k (b (.) k)^T Diag(alpha)) S
 * plus a term free of S.  Phi (dk x dk) is the product of the tokens' linear
 * parts, last first; Psi (dk x dv) is S_out for S_in = 0.  This follows from
 * the rule itself and the chunkwise form the aixai.ru blog names (section on
 * how the method is implemented in practice); the pages describe no
 * sequence-parallel split.
 * Every sequence of the call (B rows, or num_seqs packed sequences) is one
 * segment:
 *   q .. w, cu_seqlens, B .. dt : as for gdn2_chunk_fwd (the gate layout and
 *               layer prep flags apply; no S0: a segment's map does not
 *               depend on it).
 *   flags     : GDN2_FLAG_SCALAR_B / _W / _ALPHA and GDN2_FLAG_LAYER_PREP
 *               only (others return GDN2_ERR_UNSUPPORTED).
 *   Phi, Psi  : outputs, [N, H, dk, dk] and [N, H, dk, dv] float32, row-major
 *               per head.  An empty segment gives Phi = I, Psi = 0.
 *   workspace : at least gdn2_chunk_fwd_workspace_bytes(...) bytes.  On
 *               return it holds the chunks' intermediates, which
 *               gdn2_chunk_fwd with GDN2_FLAG_PREPARED reads.
 * The maps use the chunked path's arithmetic (the state rounded to dt for
 * the matrix products, as in gdn2_chunk_fwd) and accept any decay. */
gdn2_status_t gdn2_chunk_segment_map(const void *q, const void *k, const void *v, const void *alpha,
                                     const void *b, const void *w, const int32_t *cu_seqlens, int B, int T,
                                     int H, int dk, int dv, int num_seqs, int chunk, gdn2_dtype_t dt,
                                     uint32_t flags, float *Phi, float *Psi, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* The exclusive scan of G consecutive segments' maps of one sequence (H
 * heads): S_in[0] = S0, S_in[g+1] = Phi[g] S_in[g] + Psi[g], in float32.
 *   Phi, Psi  : [G, H, dk, dk] and [G, H, dk, dv] float32 (gdn2_chunk_segment_map).
 *   S0        : [H, dk, dv] float32 state entering segment 0, or NULL for zero.
 *   S_in      : output [G, H, dk, dv], the state entering every segment.
 *   S_final   : output [H, dk, dv], the state after segment G-1, or NULL.
 * Running gdn2_chunk_fwd on each segment from its S_in then gives the
 * outputs of the whole sequence.  G = 0 is allowed (S_final = S0). */
gdn2_status_t gdn2_segment_combine(const float *Phi, const float *Psi, const float *S0, int G, int H, int dk,
                                   int dv, float *S_in, float *S_final, void *stream);

/* One recurrent decode step for N sequences x H heads at constant memory
 * (aixai.ru blog: constant-memory decoding; needhelp.icu/de, section on the
 * attention bottleneck).  q, k, alpha, b are [N, H, dk]; v, w, o are
 * [N, H, dv] (element type dt); S is [N, H, dk, dv] float32 and is updated
 * in place.  o may not alias any input. */
gdn2_status_t gdn2_decode_step(const void *q, const void *k, const void *v, const void *alpha,
                               const void *b, const void *w, float *S, void *o, int N, int H,
                               int dk, int dv, gdn2_dtype_t dt, void *stream);

/* Static text of a status code. */
const char *gdn2_status_string(gdn2_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char *gdn2_last_error(void);

/* GDN2_ABI_VERSION of the loaded library. */
int gdn2_abi_version(void);

/* Kernel timing for benchmarks.  While enabled, every kernel launch made by
 * gdn2_chunk_fwd / gdn2_decode_step is bracketed by two HIP events recorded
 * on the launch stream.  gdn2_profile_read synchronises those events and
 * returns, per kernel name, the summed time in milliseconds and the launch
 * count; reset != 0 clears the record.  Enabling creates events (not device
 * memory); it is not for use under graph capture. */
gdn2_status_t gdn2_profile_enable(int on);
gdn2_status_t gdn2_profile_read(int max_kernels, const char **names, double *total_ms,
                                int *counts, int *n_kernels, int reset);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
