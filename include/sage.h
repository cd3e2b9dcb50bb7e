/*
 * sage.h -- C ABI of the MI355X (gfx950) quantized attention forward.
 *
 * The library computes the SageAttention-style forward
 *     out = softmax(Q K^T * sm_scale) V
 * in the steps the SageAttention pages describe:
 *   - smooth_k: subtract K's per-channel mean along the sequence before
 *     quantizing K ("SageAttention deployment guide", pwwt.cn, sec. 4.2 table);
 *   - Q and K quantized to INT8 with fp32 scale factors per block, per warp or
 *     per thread (deployment guide, sec. 1 first bullet and sec. 4.2
 *     qk_quant_gran); QK^T by 8-bit integer products with int32 accumulation;
 *   - softmax computed online, block by block, as in FlashAttention
 *     ("SageAttention 2.2.0 on the RX 9070 XT", pnsm.cn, sec. 2);
 *   - V kept in FP16 or lowered to FP8, P.V accumulated in fp32
 *     (deployment guide, sec. 1 second bullet, sec. 4 dispatch table and the
 *     pv_accum_dtype row of sec. 4.2); smooth_v subtracts V's mean;
 *   - output in FP16/BF16, same dtype as the inputs (deployment guide, sec. 1
 *     third bullet), optionally with the log-sum-exp (sec. 4.1 return_lse).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *   allocates nothing and keeps no state between calls, apart from the static
 *   scratch array of sage_quant_qkv_noalloc (see there).
 * - Every call is asynchronous on the caller's HIP stream (`stream`, a
 *   hipStream_t; NULL = the legacy default stream) and on the current HIP
 *   device.  Nothing is synchronised on the host.
 * - Return value: SAGE_OK (0) or a negative error code.  All argument checks
 *   run on the host before the first HIP call, so an invalid call launches
 *   nothing and writes nothing.  sage_last_error() then returns a message
 *   (thread-local, valid until the next call on the same thread).
 * - Element strides are in elements; the channel (last) dimension must be
 *   contiguous (stride 1), as the deployment guide's sec. 4.1 input rules ask.
 * - head_dim d: 1..128.  d <= 64 is zero-padded to Dp = 64, 64 < d <= 128 to
 *   Dp = 128 (deployment guide, sec. 4.1); d > 128 is SAGE_EINVAL.
 * - Grouped K/V heads (GQA): Hq must be a multiple of Hkv; query head h reads
 *   K/V head h / (Hq / Hkv) (deployment guide, sec. 4.1).
 * - Nq and Nk may differ (deployment guide, sec. 4.1).
 *
 * Quantized tensor layouts (produced by sage_quant_qk / sage_quant_v and
 * consumed by sage_attn_fwd / sage_attn_varlen_fwd):
 *   Nq_pad = round_up(Nq, 128), Nk_pad = round_up(Nk, 128); for varlen calls
 *   Nq, Nk are the maximum sequence lengths and B the number of sequences.
 *   Rows past a sequence's length and inside its last 128-row tile hold
 *   zeros; for varlen calls the tiles after that one (and their scale
 *   groups) are left unwritten -- no call reads them.
 *   q8      int8   [B][Hq ][Nq_pad][Dp]   rows >= Nq (per sequence) are 0
 *   q_scale float  [B][Hq ][Nq_pad / Gq]  Gq = 128 / 32 / 1 for
 *                                          per_block / per_warp / per_thread
 *   k8      int8   [B][Hkv][Nk_pad][Dp]
 *   k_scale float  [B][Hkv][Nk_pad / Gk]  Gk = 64 / 64 / 16
 *   k_mean  float  [B][Hkv][Dp]           written when smooth_k
 *   vt      FP8 (E4M3FN bytes) or fp16/bf16, [B][Hkv][Dp][Nk_pad]: V
 *           transposed, each aligned block of 64 keys stored in the order
 *           pos = 32*h + 16*b + 4*r + e  for key = 32*b + 8*r + 4*h + e
 *           (b in 0..1, r in 0..3, h in 0..1, e in 0..3); keys >= Nk are 0
 *   v_scale float  [B][Hkv][Dp]           FP8 only: amax_c / 448
 *   v_mean  float  [B][Hkv][Dp]           written when smooth_v
 * Quantizer (all fp32, round to nearest even): per group, scale = amax/127,
 * code = rint(x * fl32(127/amax)); all-zero group -> scale 0, codes 0.
 * V (FP8): per channel c over the sequence, code = E4M3FN(clamp(v' *
 * fl32(448/amax_c), +-448)), v' = fl32(v - v_mean_c) when smooth_v.
 * Means are fl32(fl64(exact sum) / N), independent of summation order:
 * fp16 values are summed exactly as integers in units of 2^-24 (N < 2^23);
 * bf16 values are summed in fp64, which is exact -- in any order -- when the
 * column's sum of |x| is below 2^53 u, u the smallest bf16 ulp among its
 * nonzero values (2^(floor(log2|x|) - 7), at least 2^-133): e.g. a span of
 * about 46 - log2(N) binades between its largest and smallest magnitude.
 * Beyond that the bf16 sum carries fp64 rounding and the mean can differ
 * from the exactly rounded one in its last bit.
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_OK 0
#define SAGE_EINVAL (-1)        /* invalid argument; nothing launched          */
#define SAGE_EUNSUPPORTED (-2)  /* valid request the library does not serve    */
#define SAGE_EHIP (-3)          /* a HIP runtime call or launch failed         */

#define SAGE_ABI_VERSION 1

enum sage_dtype { SAGE_F16 = 0, SAGE_BF16 = 1 };
enum sage_layout { SAGE_HND = 0, SAGE_NHD = 1 };
enum sage_gran { SAGE_PER_BLOCK = 0, SAGE_PER_WARP = 1, SAGE_PER_THREAD = 2 };
enum sage_vdtype { SAGE_V_FP8 = 0, SAGE_V_FP16 = 1 };
/* pv_accum_dtype (deployment guide, sec. 4.2: fp16 / fp32 / fp16+fp32, also
 * written fp32+fp16 and fp32+fp32 in sec. 4's dispatch table).  Every CDNA4
 * matrix instruction accumulates in fp32, so every mode accumulates P.V in
 * fp32, which is at least as accurate as the mode named. */
enum sage_pv_accum { SAGE_ACC_FP32 = 0, SAGE_ACC_FP16 = 1, SAGE_ACC_FP16_FP32 = 2, SAGE_ACC_FP32_FP32 = 3 };

/* ---------------------------------------------------------------------------
 * sage_quant_qk: smooth K (optional) and quantize Q and K to INT8.
 * Deployment guide sec. 1 (INT8 Q/K with per-block/per-thread scales) and
 * sec. 4.2 (qk_quant_gran, smooth_k).
 *
 * Inputs: q, k in `dtype`; element (b, h, n, c) of q lives at
 *   q + b*q_stride_b + h*q_stride_h + n*q_stride_n + c            (dense)
 *   q + (cu_seqlens_q[b] + n)*q_stride_n + h*q_stride_h + c       (varlen)
 * (same for k).  cu_seqlens_q/k: device int32 [B+1], non-decreasing, starting
 * at 0, or both NULL for a dense batch; with them, Nq/Nk are upper bounds on
 * every sequence length (max_seqlen) and means, groups and scales restart at
 * each sequence.
 * Outputs: q8, q_scale, k8, k_scale (layouts above); k_mean when smooth_k
 * (may be NULL otherwise).  q, q8 and q_scale all NULL: K only (for an
 * attention call that quantizes Q itself, see sage_attn_fwd).
 * workspace: device scratch of at least sage_quant_workspace_size() bytes
 * (contents need not be initialised).
 * Errors: SAGE_EINVAL for null/misaligned pointers (16-byte alignment for
 * q8, k8 and the workspace; 4-byte for scales and means), d outside 1..128,
 * B/H/N < 1, Hq % Hkv != 0, unknown enums, workspace too small.
 * ------------------------------------------------------------------------- */
typedef struct sage_quant_qk_params {
    size_t struct_size;                 /* sizeof(sage_quant_qk_params) */
    const void* q;
    const void* k;
    int dtype;                          /* enum sage_dtype */
    int B, Hq, Hkv, Nq, Nk, d;
    int64_t q_stride_b, q_stride_h, q_stride_n;
    int64_t k_stride_b, k_stride_h, k_stride_n;
    const int32_t* cu_seqlens_q;        /* device or NULL */
    const int32_t* cu_seqlens_k;        /* device or NULL */
    int gran;                           /* enum sage_gran */
    int smooth_k;                       /* 0 / 1 */
    int8_t* q8;
    float* q_scale;
    int8_t* k8;
    float* k_scale;
    float* k_mean;                      /* required when smooth_k */
    void* workspace;
    size_t workspace_bytes;
} sage_quant_qk_params;

int sage_quant_qk(const sage_quant_qk_params* p, void* stream);

/* Scratch bytes sage_quant_qk and sage_quant_v need for the exact per-channel
 * sums, for B sequences, H heads, N (max) tokens and head_dim d.  Returns 0
 * for invalid sizes. */
size_t sage_quant_workspace_size(int B, int H, int N, int d);

/* ---------------------------------------------------------------------------
 * sage_quant_v: smooth V (optional) and lay it out for the P.V product, in
 * FP8 E4M3FN with a per-channel scale, or in the input dtype.
 * Deployment guide sec. 1 second bullet (V lowered to FP8) and sec. 4.2
 * (smooth_v).
 * Inputs: v, strides and cu_seqlens_k as k in sage_quant_qk.
 * Outputs: vt (FP8 bytes when v_dtype = SAGE_V_FP8, else `dtype` elements),
 * v_scale (FP8 only), v_mean (when smooth_v).
 * Errors: as sage_quant_qk.
 * ------------------------------------------------------------------------- */
typedef struct sage_quant_v_params {
    size_t struct_size;
    const void* v;
    int dtype;
    int B, Hkv, Nk, d;
    int64_t v_stride_b, v_stride_h, v_stride_n;
    const int32_t* cu_seqlens_k;
    int v_dtype;                        /* enum sage_vdtype */
    int smooth_v;
    void* vt;
    float* v_scale;                     /* required for FP8 */
    float* v_mean;                      /* required when smooth_v */
    void* workspace;
    size_t workspace_bytes;
} sage_quant_v_params;

int sage_quant_v(const sage_quant_v_params* p, void* stream);

/* ---------------------------------------------------------------------------
 * sage_quant_qkv: sage_quant_qk and sage_quant_v in one call, with the same
 * results bit for bit, in two kernel launches instead of four (the Q tiles
 * and the K and V statistics share one launch, the K and V tiles the next).
 * The two parameter blocks are those of the separate calls; they must agree
 * on dtype, B, Hkv, Nk, d and cu_seqlens_k, and when both need a workspace
 * the two workspaces must not overlap.
 * Errors: as the separate calls, plus SAGE_EINVAL for a disagreement or
 * overlapping workspaces; nothing is launched then.
 * ------------------------------------------------------------------------- */
int sage_quant_qkv(const sage_quant_qk_params* qk, const sage_quant_v_params* v, void* stream);

/* ---------------------------------------------------------------------------
 * sage_quant_qkv_noalloc: sage_quant_qkv for callers that cannot allocate
 * device memory -- code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  Same parameters, checks, kernels and
 * results (bit for bit) as sage_quant_qkv, except that the workspace fields of
 * both parameter blocks are ignored: the exact-sum partials live in a static
 * device array of SAGE_QUANT_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends.  The call allocates nothing; its
 * first call on a device looks up that array's device address there.
 * Limit: the call needs sage_quant_qkv_noalloc_scratch_size(B, Hkv, Nk, d)
 * bytes of the array (0 for invalid sizes); beyond SAGE_QUANT_SCRATCH_BYTES
 * it returns SAGE_EINVAL and launches nothing (with the 16 MiB array: about
 * 500 sequence-heads of K/V at head_dim 128, any length).
 * Concurrency: every call on one GPU uses the same array, which keeps the last
 * call's partials (nothing in it needs to start at zero).  Calls whose work
 * overlaps on one GPU (different streams, or several host threads without
 * ordering) race on it; order them on one stream.
 * Errors: as sage_quant_qkv; SAGE_EHIP if the array's address cannot be
 * obtained.
 * ------------------------------------------------------------------------- */
#define SAGE_QUANT_SCRATCH_BYTES ((size_t)16 << 20)
size_t sage_quant_qkv_noalloc_scratch_size(int B, int Hkv, int Nk, int d);
int sage_quant_qkv_noalloc(const sage_quant_qk_params* qk, const sage_quant_v_params* v, void* stream);

/* ---------------------------------------------------------------------------
 * sage_attn_fwd: the fused attention forward on quantized operands.
 * Deployment guide sec. 1 (INT8 QK^T, FP8/FP16 P.V with fp32 accumulation,
 * FP16/BF16 output), sec. 4.1 (tensor_layout, is_causal, sm_scale default
 * 1/sqrt(head_dim), return_lse), sec. 4.2 (pv_accum_dtype); RX 9070 XT page
 * sec. 2 (blockwise softmax).
 *
 * Per query row i of (b, h): S_ij = sum_c q8_ic k8_jc (int32);
 * s_ij = S_ij * q_scale_i * k_scale_j * sm_scale (log2 domain inside); online
 * softmax over 64-key tiles in ascending key order; P rounded to FP8 (scaled
 * by 448) or to the input dtype; out = (P.V) * v_scale / l + v_mean.
 * is_causal: key j is visible to query i iff j <= i (top-left alignment).
 * lse (optional, fp32 [B][Hq][Nq]): natural-log log-sum-exp of the scores of
 * the unsmoothed K, sm_scale * q_hat_i . k_j (adds sm_scale * q_hat_i . k_mean
 * when k_mean is given).
 * out: element (b, h, n, c) at out + b*o_stride_b + h*o_stride_h +
 * n*o_stride_n + c for c < d, dtype out_dtype.
 * Q in its input precision (q non-NULL; q8 and q_scale are then not read and
 * may be NULL): the kernel quantizes each query row itself, in registers, to
 * the codes and scales sage_quant_qk would write for the same gran (neither
 * is stored), so the results are those of the q8/q_scale call bit for bit.
 * q has dtype in_dtype and the layout of sage_quant_qk's q with these
 * element strides (varlen: q_stride_b is ignored).  Accepted when
 * sage_attn_q_fusable() says so for the call's sizes, with q 16-byte aligned
 * and every stride a multiple of 8 elements.
 * Errors: SAGE_EINVAL for invalid sizes/enums/pointers (q8/k8/vt 16-byte
 * aligned), sm_scale not finite; SAGE_EUNSUPPORTED for q given on a call that
 * sage_attn_q_fusable() rejects.
 * ------------------------------------------------------------------------- */
typedef struct sage_attn_params {
    size_t struct_size;
    const int8_t* q8;
    const float* q_scale;
    const int8_t* k8;
    const float* k_scale;
    const float* k_mean;                /* NULL: K was not smoothed (no LSE term) */
    const void* vt;
    const float* v_scale;               /* FP8 only */
    const float* v_mean;                /* NULL: V was not smoothed */
    int B, Hq, Hkv, Nq, Nk, d;
    int gran;                           /* must match sage_quant_qk */
    int v_dtype;                        /* enum sage_vdtype */
    int pv_accum;                       /* enum sage_pv_accum (all fp32 here) */
    int is_causal;
    float sm_scale;                     /* <= 0: 1/sqrt(d) */
    int in_dtype;                       /* dtype q/k/v had (P precision on the FP16 path) */
    void* out;
    int out_dtype;                      /* enum sage_dtype */
    int64_t o_stride_b, o_stride_h, o_stride_n;
    float* lse;                         /* NULL: no LSE */
    const void* q;                      /* NULL: q8 / q_scale are the query operand */
    int64_t q_stride_b, q_stride_h, q_stride_n;
} sage_attn_params;

int sage_attn_fwd(const sage_attn_params* p, void* stream);

/* sage_attn_q_fusable: 1 if an attention call (sage_attn_fwd, its varlen and
 * split-KV forms) with these sizes takes Q in its input precision, else 0.
 * It does when V is FP8 (the kernel with a 256-row query tile), head_dim is a
 * multiple of 8 above 64 (128 padded channels), and the query tile's
 * quantization groups lie inside one
 * head: always for dense or varlen rows of one head per tile; with the query
 * heads of a K/V head packed into one tile (grouped heads, non-causal, dense,
 * Nq <= 128) per_warp needs Nq % 32 == 0 and per_block Nq % 128 == 0. */
int sage_attn_q_fusable(int B, int Hq, int Hkv, int Nq, int d, int gran, int v_dtype, int is_causal, int varlen);

/* ---------------------------------------------------------------------------
 * sage_attn_varlen_fwd: as sage_attn_fwd for a packed batch of sequences
 * (deployment guide sec. 4.2, sageattn_varlen with cu_seqlens_q/k).  The
 * quantized operands use the layouts above with B = number of sequences and
 * Nq/Nk = max_seqlen_q/k.  Causal masking is per sequence.  A sequence longer
 * than max_seqlen (here and in the quantize calls) is cut to its first
 * max_seqlen tokens, all that its padded slot holds: later keys are ignored
 * and the outputs and LSEs of later queries are not written.  out is packed
 * token-major: token (cu_seqlens_q[b] + n), head h, channel c at
 * out + (cu_seqlens_q[b] + n)*o_stride_n + h*o_stride_h + c.
 * lse (optional): fp32 [Hq][total_q], total_q = cu_seqlens_q[B].
 * ------------------------------------------------------------------------- */
typedef struct sage_attn_varlen_params {
    sage_attn_params base;              /* o_stride_b is ignored */
    const int32_t* cu_seqlens_q;        /* device int32 [B+1] */
    const int32_t* cu_seqlens_k;        /* device int32 [B+1] */
    int total_q;                        /* cu_seqlens_q[B] (for the LSE layout) */
} sage_attn_varlen_params;

int sage_attn_varlen_fwd(const sage_attn_varlen_params* p, void* stream);

/* ---------------------------------------------------------------------------
 * sage_debug_qk_scores: the int32 scores S = q8 k8^T of the attention kernel's
 * own QK^T tile code, for checking them exactly.  mode 0: full dump,
 * scores int32 [B][Hq][Nq][Nk]; mode 1: per-row checksums, int64
 * [B][Hq][Nq][2] = (sum_j S_ij, sum_j (j+1) S_ij) modulo 2^64.  Dense only.
 * Errors: as sage_attn_fwd.
 * ------------------------------------------------------------------------- */
int sage_debug_qk_scores(const sage_attn_params* p, int mode, void* scores, void* stream);

/* sage_debug_qk_scores_varlen: the per-row checksums of mode 1 for a packed
 * varlen batch (sage_attn_varlen_params; out, lse and the V fields are not
 * used), from the same tile code, per sequence with the forward's lengths:
 * checksums int64 [Hq][total_q][2] = (sum_j S_ij, sum_j (j+1) S_ij) modulo
 * 2^64 over the keys j of row i's own sequence.
 * Errors: SAGE_EINVAL for invalid sizes, NULL or misaligned pointers,
 * total_q < 1. */
int sage_debug_qk_scores_varlen(const sage_attn_varlen_params* p, void* checksums, void* stream);

/* ---------------------------------------------------------------------------
 * sage_attn_fwd_splitkv: sage_attn_fwd for few queries against many keys
 * (deployment guide sec. 4.1: q and k/v lengths may differ, e.g. encoder-
 * decoder attention or decoding against a long context), where one workgroup
 * per 256-query tile would leave most of the GPU idle.  The keys are cut into
 * ranges of split_len = round_up(ceil(Nk / n_splits), 128) keys (the last one
 * shorter; ranges that would be empty are dropped, so S = ceil(Nk /
 * split_len) <= n_splits).  Each range runs the same online softmax as
 * sage_attn_fwd, starting afresh at its first key; its normalised output is
 * stored in fp32 with its log-sum-exp in the workspace, and the S partial
 * results are then combined as sage_merge_states does (in fp32, one rounding
 * to out_dtype at the end).  With S = 1 the result is bit-identical to
 * sage_attn_fwd.
 * Same parameters and layouts as sage_attn_fwd; non-causal only.
 * workspace: device memory, 256-byte aligned, of at least
 * sage_attn_splitkv_workspace_size(B, Hq, Nq, Nk, d, n_splits) bytes (0 for
 * invalid sizes); it holds S x [B][Hq][Nq][d] fp32 outputs and S x [B][Hq][Nq]
 * fp32 LSEs and need not be initialised.
 * Errors: as sage_attn_fwd; SAGE_EINVAL for n_splits outside 1..64 or a
 * missing, misaligned or too small workspace; SAGE_EUNSUPPORTED for
 * is_causal.
 * ------------------------------------------------------------------------- */
size_t sage_attn_splitkv_workspace_size(int B, int Hq, int Nq, int Nk, int d, int n_splits);
int sage_attn_fwd_splitkv(const sage_attn_params* p, int n_splits, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---------------------------------------------------------------------------
 * sage_merge_states: combine attention results computed over S disjoint key
 * sets of the same queries, using the log-sum-exp each one returned
 * (deployment guide sec. 4.1: return_lse, for Ring-Attention-style use).
 * With o_s the normalised output of key set s and L_s its natural-log LSE,
 * the attention over all keys is out = sum_s exp(L_s - L) o_s and
 * L = log sum_s exp(L_s), exactly in real arithmetic.
 * Computed per row in fp32: m = max_s L_s, w_s = exp(L_s - m) (0 when
 * L_s = -inf), W = sum_s w_s, out = sum_s (w_s / W) o_s rounded once to the
 * output dtype (nearest even), L = m + log W.  A row whose S values are all
 * -inf (it saw no key) gives out = 0 and L = -inf.  Sums run s = 0 .. S-1.
 * parts: S fp16/bf16 results, element (s, b, h, n, c) at parts + s*ps_s +
 * b*ps_b + h*ps_h + n*ps_n + c for c < d; the output row (b, h, n) at out +
 * b*o_stride_b + h*o_stride_h + n*o_stride_n.  lse_parts is fp32
 * [S][B][H][N] contiguous (what sage_attn_fwd writes for each set, stacked);
 * lse (optional) receives fp32 [B][H][N].  out must not overlap the inputs.
 * Sizes: 1 <= S <= 64, 1 <= d <= 1024, B, H, N >= 1.
 * Errors: SAGE_EINVAL for invalid sizes or dtype, NULL parts/lse_parts/out,
 * or pointers not aligned to their element size.
 * ------------------------------------------------------------------------- */
typedef struct sage_merge_params {
    size_t struct_size;
    int n_parts;                        /* S */
    int dtype;                          /* enum sage_dtype: parts and out */
    int B, H, N, d;
    const void* parts;
    int64_t ps_s, ps_b, ps_h, ps_n;     /* element strides of parts */
    const float* lse_parts;             /* [S][B][H][N] */
    void* out;
    int64_t o_stride_b, o_stride_h, o_stride_n;
    float* lse;                         /* NULL: no merged LSE */
} sage_merge_params;

int sage_merge_states(const sage_merge_params* p, void* stream);

const char* sage_last_error(void);
int sage_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H */
