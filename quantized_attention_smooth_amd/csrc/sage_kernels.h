// sage_kernels.h -- kernel argument blocks and host launch helpers shared by
// the C-ABI layer (sage_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

// Tile sizes.  One attention workgroup of 4 wavefronts covers kBQ query rows
// (64 per wavefront: two MFMA column blocks); the key loop advances kBK keys
// per step, which is also the online-softmax tile.  Quantized rows are padded
// to kPad.
constexpr int kBQ = 256;
constexpr int kBK = 64;
constexpr int kPad = 128;
constexpr int kThreads = 256;

// Per-channel statistics pass over K or V (exact sums; min/max for V).
struct StatsArgs {
    const void* x;
    int64_t sb, sh, sn;          // element strides (batch, head, token)
    const int32_t* cu;           // varlen offsets or nullptr
    int B, H, N, d, dp;          // N: dense length or max length
    int chunks;                  // token chunks per (b, h)
    int chunk_len;               // tokens per chunk (a multiple of kStatsChunk)
    int want_minmax;
    void* part_sum;              // [B][H][chunks][dp] int64 (fp16) or double (bf16)
    float* part_min;             // [B][H][chunks][dp]
    float* part_max;
    int smooth;                  // V: amax over |v - mean| (else over |v|)
    float* out_mean;             // caller's k_mean / v_mean, or nullptr
    float* out_scale;            // caller's v_scale, or nullptr
};

// INT8 quantization of Q or K rows.
struct QuantRowsArgs {
    const void* x;
    int64_t sb, sh, sn;
    const int32_t* cu;
    int B, H, N, npad, d;
    int group_shift;             // log2(rows per scale group)
    int8_t* out;                 // [B][H][npad][dp]
    float* scale;                // [B][H][npad >> group_shift]
};

// Transposed V operand (FP8 codes or fp16/bf16).
struct QuantVArgs {
    const void* v;
    int64_t sb, sh, sn;
    const int32_t* cu;
    int B, H, N, npad, d;
    void* vt;                    // [B][H][dp][npad]
};

struct AttnArgs {
    const int8_t* q8;
    const float* qs;
    const int8_t* k8;
    const float* ks;
    const float* kmean;
    const void* vt;
    const float* vs;
    const float* vmean;
    void* out;
    float* lse;
    const int32_t* cu_q;
    const int32_t* cu_k;
    int B, Hq, Hkv, Nq, Nk, d;
    int nq_pad, nk_pad;
    int gq_shift, gk_shift;
    int causal;
    float sm_scale;
    int64_t ob, oh, on;
    int out_vec4;                // 4 consecutive channels may be stored as one 8-byte (16-byte fp32) write
    int out_vec8;                // 16-bit output whose rows take 16-byte writes of 8 channels (d % 8 == 0)
    int out_f32;                 // out holds fp32 values (split-KV partial results), strides in floats
    int lse_varlen;              // LSE layout [Hq][total_q] instead of [B][Hq][Nq]
    int total_q;
    int n_qtiles;                // query tiles per (b, h)
    int num_wg;
    // split-KV (dense, non-causal): workgroup split s of a query tile
    // covers keys [s * split_len, min(Nk, (s + 1) * split_len)) and writes its
    // output and LSE split_out / split_lse elements after split 0's
    int pack_gqa;                // FP8 V, non-causal, dense only: rows of all query heads of a K/V head together
    int n_splits;                // 1: no split
    int split_len;               // multiple of 128
    int64_t split_out, split_lse;
    // debug score dump (sage_debug_qk_scores)
    void* dbg;
    int dbg_mode;
    // Q in its input precision instead of q8 / qs (nullptr: not given); the
    // kernel quantizes it.  Element strides; varlen rows at (cu_q[b] + n) * qsn.
    const void* qraw;
    int64_t qsb, qsh, qsn;
    int q_bf16;
};

// Merge of partial attention results over disjoint key sets (merge.hip).
struct MergeArgs {
    const void* parts;           // part s, row (b, h, n), channel c at parts + s*ps + b*pb + h*ph + n*pn + c
    int64_t ps, pb, ph, pn;
    const float* lse_parts;      // [S][B][H][N], natural log
    void* out;                   // row (b, h, n) at out + b*ob + h*oh + n*on
    int64_t ob, oh, on;
    float* lse;                  // [B][H][N] or null
    int S, B, H, N, d;
    int parts_f32;               // parts are fp32 (split-KV partials) instead of the output dtype
};

// Launchers (defined in the kernel translation units).  Each returns the
// hipError_t of the launch.
// Q and K: Q tiles and the K statistics (smooth) in one launch, then the K
// tiles; without smoothing, one launch for both.
hipError_t launch_quant_qk(const QuantRowsArgs& q, const QuantRowsArgs& k, const StatsArgs& ks, bool smooth,
                           bool bf16, bool vec, hipStream_t s);
// V: statistics (when stats), then the tiles.
hipError_t launch_quant_v(const QuantVArgs& a, const StatsArgs& vs, bool stats, bool smooth, bool bf16, bool fp8,
                          bool vec, hipStream_t s);
// Q, K and V together in two launches; ks and vs must use disjoint
// workspaces.
hipError_t launch_quant_qkv(const QuantRowsArgs& q, const QuantRowsArgs& k, const StatsArgs& ks, bool smooth_k,
                            const QuantVArgs& v, const StatsArgs& vs, bool v_stats, bool bf16, bool fp8, bool vec,
                            hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, int dp, int pv /*0 fp8, 1 fp16, 2 bf16*/, bool out_bf16,
                       hipStream_t s);
hipError_t launch_qk_scores(const AttnArgs& a, int dp, hipStream_t s);
// vec: d % 8 == 0 and every part/out row start 16-byte aligned (8 channels per thread)
hipError_t launch_merge(const MergeArgs& a, bool bf16, bool vec, hipStream_t s);

// Statistics chunks: kStatsChunk tokens, or longer for long sequences so
// that a (b, h) has at most kMaxChunks partials (every tile workgroup of the
// quantize pass reduces all partials of its (b, h)).
constexpr int kStatsChunk = 256;
// Query heads sharing a K/V head are packed into one workgroup's rows when
// each has at most this many queries.
constexpr int kPackMaxNq = 128;
constexpr int kMaxChunks = 32;

}  // namespace sage
