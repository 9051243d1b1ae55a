/*
 * sdpa_math — materialised-probability scaled-dot-product attention forward
 * for AMD Instinct MI355X (gfx950).
 *
 * One call returns the attention output O, the full probability map P and
 * the float32 row log-sum-exp LSE. This is the math-backend contract of the
 * FlagOS-OP pull request "feat: add sdpa_math operator (Ascend Triton + P800
 * exact-P/A1)" (Overview: the operator returns (out, attn_probs) for callers
 * that must see the probabilities), with the row-wise LSE of its "P800
 * exact-P fast path" update (P = exp(scale * Q K^T - LSE)).
 *
 * For every batch b, query head h, query row i and key j, with
 * g = Hq / Hkv and kv head h' = h / g:
 *   s_ij = scale * sum_d Q[b,h,i,d] * K[b,h',j,d]
 *   s_ij = -inf  if causal and j > i + c (c = 0: top-left alignment;
 *                c = Skv - Sq: bottom-right, the last query row keeps every
 *                key), or if a boolean
 *                mask holds False at (b,h,i,j); s_ij += mask[b,h,i,j] for an
 *                additive mask (masks broadcast over size-1 dimensions)
 *   LSE_i  = log sum_j exp(s_ij)            (-inf when every key is removed)
 *   P_ij   = exp(s_ij - LSE_i)              (0 on rows whose LSE is -inf)
 *   O_i    = sum_j P_ij * V[b,h',j,:]       (0 on rows whose LSE is -inf)
 * Semantics fixed by that page's Implementation section (fully-masked rows
 * give P = O = 0, head counts that do not divide are an error, causal and an
 * explicit mask are exclusive) and its Intentional-divergences section (a
 * boolean mask removes keys with -inf). Dead rows report LSE = -inf and LSE is
 * laid out [B, H, S] in float32, as the cudnn-frontend pull request "[SDPA]
 * SM80 fwd: TemplateParams kernels, plan-time compile, sym_int THD extents"
 * records in its merge-log notes.
 *
 * Numerics: scores, row statistics and the P·V accumulation run in float32;
 * P is rounded to the output dtype with round-to-nearest-even. O accumulates
 * the float32 probabilities, carried into the 16-bit matrix products as the
 * stored rounded value plus its rounded residual (twice the dtype's
 * precision), so O is the float32 sum of P·V rounded once to the dtype: the
 * FlagOS-OP page's Validation section reports worst errors of half a unit of
 * the output dtype, which only a correctly rounded O reaches.
 */
#ifndef SDPA_MATH_H
#define SDPA_MATH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDPA_MATH_VERSION 1

typedef enum {
    SDPA_F32 = 0,
    SDPA_F16 = 1,
    SDPA_BF16 = 2,
    SDPA_BOOL = 3 /* one byte per element, 0 = False */
} sdpa_dtype_t;

/*
 * A strided view of device memory. `ndim` is 4 for q, k, v, out, probs and
 * the mask (a mask of fewer dims is passed right-aligned with leading size-1
 * dims), and 3 for lse. Sizes and strides are in ELEMENTS; a size-1 dim may
 * have any stride. The library never takes ownership of `data`.
 */
typedef struct {
    void* data;
    int32_t dtype; /* sdpa_dtype_t */
    int32_t ndim;
    int64_t sizes[4];
    int64_t strides[4];
} sdpa_tensor_t;

typedef enum {
    SDPA_OK = 0,
    SDPA_ERR_INVALID_ARG = 1, /* shapes, dtypes, null pointers, semantic rule broken */
    SDPA_ERR_UNSUPPORTED = 2, /* valid call the library does not implement (layout, head dim) */
    SDPA_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
} sdpa_status_t;

typedef enum {
    SDPA_PATH_AUTO = 0,    /* choose by the number of score tiles (see sdpa_math_plan) */
    SDPA_PATH_FUSED = 1,   /* one sweep over the keys; scores stay on chip */
    SDPA_PATH_TWOPASS = 2, /* row statistics sweep, then a probability/output sweep */
    SDPA_PATH_FUSED_WIDE = 3 /* reported by sdpa_math_plan only: the fused path on its
                                wide kernel (several 32-row groups per workgroup) */
} sdpa_path_t;

/*
 * sdpa_math_fwd — enqueue the forward on `hip_stream` (a hipStream_t; NULL =
 * the null stream) and return without synchronising.
 *
 * q      [B, Hq, Sq, D]   f32 | f16 | bf16
 * k      [B, Hkv, Skv, D] same dtype as q
 * v      [B, Hkv, Skv, Dv] same dtype as q; Dv == D in this version
 * mask   NULL, or a bool or q-dtype tensor broadcastable to [B, Hq, Sq, Skv]
 *        (bool: True keeps the key; float: added to the scaled score)
 * is_causal  0: no causal mask; 1: top-left causal; 2: bottom-right causal
 *        (query i keeps keys j <= i + Skv - Sq: the alignment of a query chunk
 *        against a longer key cache, named by the cudnn-frontend merge-log
 *        notes; when Sq > Skv the first Sq - Skv rows keep no key and are dead
 *        rows). Exclusive with `mask`; other values are INVALID_ARG.
 * scale  multiplier of Q K^T (the Python layer passes 1/sqrt(D) by default,
 *        as the cudnn-frontend merge-log notes resolve a missing scale)
 * enable_gqa nonzero lets Hq be a multiple of Hkv; query head h then reads
 *        kv head h / (Hq / Hkv)
 * out    [B, Hq, Sq, Dv] q dtype     (written)
 * probs  [B, Hq, Sq, Skv] q dtype    (written in full, zeros included)
 * lse    [B, Hq, Sq] f32             (written)
 *
 * Layout: every tensor needs stride 1 in its last dim (a broadcast mask may
 * use stride 0 there); q, k, v need a 16-byte-aligned base and strides that
 * are multiples of 16 bytes (the operand contract of the cudnn-frontend page,
 * merge-log note on dense operands). Outputs may be uninitialised.
 * Ownership: the caller allocates every buffer; the library allocates no
 * device memory, keeps no device state between calls, never synchronises and
 * never reads device data on the host. Calls on different streams may run
 * concurrently.
 * Errors: validation runs before any launch; on error nothing is enqueued and
 * sdpa_math_last_error() describes the problem. Head dims 32, 64 and 128 are
 * implemented; others give SDPA_ERR_UNSUPPORTED. An empty problem (B*Hq*Sq
 * == 0) is SDPA_OK with nothing launched; Skv == 0 yields O = 0, LSE = -inf.
 */
sdpa_status_t sdpa_math_fwd(const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                            const sdpa_tensor_t* v, const sdpa_tensor_t* mask,
                            int is_causal, float scale, int enable_gqa,
                            sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse,
                            void* hip_stream);

/*
 * sdpa_math_fwd_path — sdpa_math_fwd with the path forced (SDPA_PATH_AUTO
 * behaves exactly like sdpa_math_fwd): the per-call form of the forced
 * on/off/auto switch of the FlagOS-OP page's single-kernel fusion update
 * (an experiment knob there, as here). A forced path the shape cannot take
 * (the fused path needs every processed key row of a query block to fit on
 * chip) returns SDPA_ERR_UNSUPPORTED with nothing launched; any other path
 * value is SDPA_ERR_INVALID_ARG. Both paths compute the same values within
 * the stated tolerances; arguments, layout, ownership and errors otherwise
 * as sdpa_math_fwd.
 */
sdpa_status_t sdpa_math_fwd_path(const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                                 const sdpa_tensor_t* v, const sdpa_tensor_t* mask,
                                 int is_causal, float scale, int enable_gqa,
                                 sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse,
                                 void* hip_stream, int path);

/*
 * sdpa_math_workspace_bytes — bytes of device workspace with which
 * sdpa_math_fwd_ws splits the keys of this call over more workgroups (0: it
 * would not split). Splitting pays when there are few query rows per key
 * (decode, a short query chunk against a long key cache): each query block's
 * keys are cut into ranges whose row statistics and float32 partial outputs
 * go to the workspace, combined into the same O, P and LSE (the FlagOS-OP
 * "P800 exact-P fast path" update: P = exp(S - LSE) with the row LSE folded
 * from the ranges' statistics). Where fewer bytes move that way (roughly: 8
 * times the query rows per key head below D times the element size), the
 * ranges run in one sweep over the keys on the wide fused kernel and the
 * workspace also holds every probability as float32, relative to its
 * range's row maximum, until a combine launch scales it into P; otherwise
 * the two-pass kernel runs a statistics and a probability launch per range.
 * Validates like sdpa_math_plan; *bytes is set to 0 on error.
 */
sdpa_status_t sdpa_math_workspace_bytes(const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                                        const sdpa_tensor_t* v, const sdpa_tensor_t* mask,
                                        int is_causal, int enable_gqa, size_t* bytes);

/*
 * sdpa_math_fwd_ws — sdpa_math_fwd_path with a caller-owned device workspace
 * (256-byte aligned, at least sdpa_math_workspace_bytes, or NULL). The
 * library still allocates nothing; with a NULL or too small workspace the
 * call runs unsplit. The workspace is scratch for this call only (its
 * contents afterwards are unspecified); calls that share a workspace must be
 * ordered on one stream.
 */
sdpa_status_t sdpa_math_fwd_ws(const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                               const sdpa_tensor_t* v, const sdpa_tensor_t* mask,
                               int is_causal, float scale, int enable_gqa,
                               sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse,
                               void* workspace, size_t workspace_bytes, void* hip_stream, int path);

/*
 * sdpa_math_fwd_dropout — sdpa_math_fwd with dropout applied to P under one
 * of the two rules the FlagOS-OP page fixes (Implementation section: the
 * explicit and the random dropout rule; Intentional divergences: with
 * dropout_p > 0 the output is the dropped probabilities times V; single-
 * kernel fusion update: dropout always takes the two-stage path):
 *   rule 0 (explicit keep-mask): probs = keep * P,            out = (keep * P) V / (1 - dropout_p)
 *   rule 1 (random):             probs = keep * P / (1 - p),  out = probs V
 * with P, LSE (of the undropped softmax) and the masking as sdpa_math_fwd.
 * keep   bool, broadcastable to [B, Hq, Sq, Skv] (True keeps the entry): the
 *        random numbers of the call, drawn by the caller (for rule 1, keep
 *        with probability 1 - dropout_p); read only
 * dropout_p  in [0, 1), else SDPA_ERR_INVALID_ARG; rule 0 or 1, else
 *        SDPA_ERR_INVALID_ARG
 * Runs the two-pass kernel (two compute waves and a loader wave), never the
 * fused path nor key ranges. Other arguments, layout, ownership and errors as
 * sdpa_math_fwd.
 */
sdpa_status_t sdpa_math_fwd_dropout(const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                                    const sdpa_tensor_t* v, const sdpa_tensor_t* mask,
                                    int is_causal, float scale, int enable_gqa,
                                    float dropout_p, const sdpa_tensor_t* keep, int rule,
                                    sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse,
                                    void* hip_stream);

/*
 * sdpa_math_fwd_varlen — the forward over packed variable-length sequences
 * (the THD layout with cumulative sequence offsets that the cudnn-frontend
 * pull request "[SDPA] SM80 fwd: TemplateParams kernels, plan-time compile,
 * sym_int THD extents" serves: token-major (T, H, D) tensors plus
 * cu_seqlens). Sequence b holds query tokens cu_seqlens_q[b] ..
 * cu_seqlens_q[b+1] and key/value tokens cu_seqlens_kv[b] ..
 * cu_seqlens_kv[b+1]; it attends only within itself, with the semantics of
 * sdpa_math_fwd (is_causal 1: top-left, 2: bottom-right, per sequence).
 * q    [Tq, Hq, D];  k [Tkv, Hkv, D];  v [Tkv, Hkv, Dv]   (3 dims, last contiguous)
 * cu_seqlens_q, cu_seqlens_kv  device int32 arrays of n_seqs + 1 offsets,
 *      non-decreasing from 0 (read on the device only: the host never reads
 *      them; offsets outside [0, T] are clamped to the tensors)
 * max_seqlen_q, max_seqlen_kv  upper bounds of the sequences' lengths (the
 *      launch grid covers max_seqlen_q query rows per sequence; longer
 *      sequences are cut to the bounds)
 * out   [Tq, Hq, Dv] q dtype; probs [Tq, Hq, max_seqlen_kv] q dtype: row t of
 *      head h holds the probabilities over its own sequence's keys in entries
 *      0 .. len_kv - 1 and zeros in the rest; lse [Tq, Hq] f32
 * No attention mask (causal only), no dropout; the two-pass kernel. Other
 * arguments, ownership and errors as sdpa_math_fwd.
 */
sdpa_status_t sdpa_math_fwd_varlen(const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                                   const sdpa_tensor_t* v, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_kv, int64_t n_seqs,
                                   int64_t max_seqlen_q, int64_t max_seqlen_kv, int is_causal,
                                   float scale, int enable_gqa, sdpa_tensor_t* out,
                                   sdpa_tensor_t* probs, sdpa_tensor_t* lse, void* hip_stream);

/*
 * sdpa_math_fwd_noalloc — sdpa_math_fwd_ws for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): no workspace argument and nothing allocated. A
 * call whose keys the planner splits into ranges keeps the ranges' row
 * statistics and float32 partial outputs in a static scratch array of
 * SDPA_MATH_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on, until the process ends (its device address is looked up once per
 * device, on the first call there). One-sweep ranges that would need more
 * than that run as the two-pass split instead; a two-pass split that would
 * need more returns SDPA_ERR_UNSUPPORTED before any launch (sdpa_math_fwd_ws
 * with a caller workspace takes it); no part of the scratch needs to start
 * at zero.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents: calls that may overlap on one GPU (different streams,
 * threads) race and must be ordered by the caller. Arguments, layout,
 * outputs and the other errors as sdpa_math_fwd_path.
 */
#define SDPA_MATH_NOALLOC_SCRATCH_BYTES (32u << 20)
sdpa_status_t sdpa_math_fwd_noalloc(const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                                    const sdpa_tensor_t* v, const sdpa_tensor_t* mask,
                                    int is_causal, float scale, int enable_gqa,
                                    sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse,
                                    void* hip_stream, int path);

/*
 * sdpa_math_plan — validate the shapes exactly as sdpa_math_fwd would and
 * report, without launching anything:
 *   *path         the path SDPA_PATH_AUTO resolves to in a call with its
 *                 workspace (sdpa_math_fwd_ws; SDPA_PATH_FUSED_WIDE when that
 *                 is the fused path on its wide kernel, key ranges included;
 *                 a call that the planner splits over key ranges runs
 *                 unsplit without a workspace)
 *   *tiles_per_bh score tiles one (batch, head) processes with this
 *                 library's tiling, after causal truncation
 *   *tiles_64     the same count in 64x64 tiles (the unit of the FlagOS-OP
 *                 page's fused-vs-two-stage rule, single-kernel fusion update)
 * out/probs/lse may be NULL here. Any output pointer may be NULL.
 * SDPA_PATH_AUTO (thresholds measured on MI355X): where the fused path's
 * wide kernel can hold the keys of a non-causal call, the fused path when
 * the call has a mask, Skv >= 512 and Sq <= 256, or no mask, Skv >= 1024
 * and Sq <= 128; otherwise the fused path when it can hold the keys,
 * Sq <= 128, tiles_64 <= 64, (is_causal or Skv >= 512) and no additive mask
 * over more than 64 rows; else the two-pass path. The environment variable
 * SDPA_MATH_PATH=auto|fused|twopass forces the choice;
 * SDPA_MATH_FUSED_MAX_ROWS=<n>, SDPA_MATH_FUSED_MAX_TILES=<n> and
 * SDPA_MATH_FUSED_MIN_KEYS=<n> move the three thresholds of the second
 * rule; SDPA_MATH_FUSED_WIDE=0 keeps the fused path off its wide kernel,
 * =1 on it (SDPA_ERR_UNSUPPORTED where it cannot hold the keys).
 * With a workspace (sdpa_math_fwd_ws, sdpa_math_fwd_noalloc), under
 * SDPA_PATH_AUTO: a call of one to four query rows (32 * Sq <= D times the
 * element size) that the whole-call wide kernel does not take runs its keys
 * as ranges in one sweep on the wide kernel, then a combine launch (the
 * query heads of a KV group sharing a workgroup); other calls with few
 * query blocks against many keys run the two-pass kernel over key ranges.
 * SDPA_MATH_RANGES=0 keeps the one-sweep ranges off, =1 takes them wherever
 * they fit; SDPA_MATH_SPLITS=<n> forces n two-pass ranges.
 * On the two-pass path, a non-causal grouped-head call (query heads per KV
 * head a multiple of 4) without a mask or with one that all query heads
 * share runs four query heads of a KV group per workgroup on 32 shared rows;
 * SDPA_MATH_HEAD_ROWS=0 keeps one head per workgroup. Outputs do not depend
 * on either choice.
 */
sdpa_status_t sdpa_math_plan(const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                             const sdpa_tensor_t* v, const sdpa_tensor_t* mask,
                             int is_causal, int enable_gqa,
                             int32_t* path, int64_t* tiles_per_bh, int64_t* tiles_64);

/*
 * sdpa_math_bwd — the backward of sdpa_math_fwd: gradients of q, k and v
 * for a loss whose gradients with respect to the two outputs are `dout`
 * (dL/dO) and `dprobs` (dL/dP; NULL when no gradient reaches P). This is the
 * two-output gradient of the FlagOS-OP page's Implementation section (its
 * autograd.Function takes both) and of its "P800 fused backward" update (the
 * softmax Jacobian taken from the probabilities; the gradients of the query
 * heads that share a key/value head summed back onto it):
 *   P_ij  = exp(S_ij - LSE_i)        (S as in sdpa_math_fwd; recomputed from
 *                                     the saved LSE, not read back)
 *   dP_ij = dout_i . v_j + dprobs_ij
 *   dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
 *   dq_i  = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 *   dv_j  = sum_i P_ij dout_i        (i over every query head of the group)
 * Removed keys and dead rows receive no gradient; no gradient is returned for
 * an additive mask.
 *
 * q, k, v, mask, is_causal, scale, enable_gqa: exactly as passed to the
 *        forward (same values: the probabilities are recomputed from them)
 * lse    [B, Hq, Sq] f32, the forward's LSE
 * dout   [B, Hq, Sq, Dv] q dtype; dprobs [B, Hq, Sq, Skv] q dtype or NULL
 * dq     [B, Hq, Sq, D], dk [B, Hkv, Skv, D], dv [B, Hkv, Skv, Dv]: q dtype,
 *        written in full (may be uninitialised)
 * workspace  device memory of at least sdpa_math_bwd_workspace_bytes bytes,
 *        16-byte aligned, owned by the caller, scratch for this call only
 *        (calls sharing one must be ordered on a stream)
 * Layout: last dims contiguous; q, k, v, dout, dq, dk, dv need 16-byte
 * aligned bases and row strides. Errors as sdpa_math_fwd, plus
 * SDPA_ERR_INVALID_ARG for a missing or short workspace; nothing is enqueued
 * on error. Enqueued on `hip_stream` without synchronising; deterministic
 * (no atomics). The library allocates nothing.
 */
sdpa_status_t sdpa_math_bwd(const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                            const sdpa_tensor_t* v, const sdpa_tensor_t* mask,
                            int is_causal, float scale, int enable_gqa,
                            const sdpa_tensor_t* lse, const sdpa_tensor_t* dout,
                            const sdpa_tensor_t* dprobs, sdpa_tensor_t* dq, sdpa_tensor_t* dk,
                            sdpa_tensor_t* dv, void* workspace, size_t workspace_bytes,
                            void* hip_stream);

/*
 * sdpa_math_bwd_workspace_bytes — bytes of workspace sdpa_math_bwd needs for
 * these inputs: one float32 per query row (4 * B * Hq * Sq, rounded up to
 * 256), plus, for a causal call whose key blocks (64 keys) number fewer
 * than 1024, float32 partial dk and dv for each of up to 4 query ranges
 * (8 * ranges * B * Hkv * Skv * D). Validates the inputs like
 * sdpa_math_plan; *bytes is 0 on error.
 */
sdpa_status_t sdpa_math_bwd_workspace_bytes(const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                                            const sdpa_tensor_t* v, const sdpa_tensor_t* mask,
                                            int is_causal, int enable_gqa, size_t* bytes);

/* Message of the last failed call on this thread ("" if none): the text
 * behind the status codes above, which map the FlagOS-OP page's
 * Implementation-section error rules (heads that do not divide, causal with
 * a mask). The string is owned by the library and valid until the next call
 * on the same thread; never NULL. */
const char* sdpa_math_last_error(void);

/* SDPA_MATH_VERSION of the loaded library (the C ABI above; a caller built
 * against another version should not use the library). Never fails. */
int sdpa_math_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MATH_H */
