// quant.hip -- HBM-bound quantize passes for the quantized attention forward
// (gfx950).
//
//   statistics       exact per-channel sums of K or V along the sequence
//                    (plus min/max for FP8 V), one workgroup per 256-token
//                    chunk of one (sequence, head), written as partials;
//   row quantization Q or K rows -> INT8 codes + one fp32 scale per group of
//                    rows (per_block / per_warp / per_thread);
//   V quantization   V -> transposed FP8 E4M3FN codes (or fp16/bf16), keys
//                    reordered inside each 64-key block for the P.V MFMA.
// Four launches in all: [Q rows + K statistics], [K rows], [V statistics],
// [V].  Every workgroup of the K / V pass reduces the (at most kMaxChunks)
// chunk partials of its (sequence, head) itself -- they sit in L2 -- after
// issuing its own loads, so no separate finalize pass (and no cross-workgroup
// synchronisation, whose device-scope fences write back and invalidate the
// per-XCD L2) is needed.
//
// Method ("SageAttention deployment guide", pwwt.cn): sec. 1 first bullet
// (Q, K -> INT8 with per-block / per-thread scale factors), second bullet
// (V -> FP8), sec. 4.2 (qk_quant_gran; smooth_k subtracts K's mean along the
// sequence; smooth_v subtracts V's mean).
//
// Bit-exactness: a mean is fl32(fl64(exact sum) / N).  fp16 inputs are
// summed as multiples of 2^-24 (every fp16 value is one): each thread adds
// its 16 values in fp64, which is exact (|sum| < 2^44 units), and the
// threads' and chunks' sums are combined as int64 (exact for N < 2^23).
// bf16 inputs are summed in fp64, which is exact -- and therefore independent
// of the summation order -- when the column's sum of |x| is below 2^53 times
// the smallest bf16 ulp among its nonzero values (every partial sum is then a
// multiple of that ulp that fp64 holds exactly).  The quantizer's fp32 operations are single
// IEEE operations (no contraction), so codes and scales are reproducible.
#include <type_traits>

#include "sage_device.h"

#pragma clang fp contract(off)

namespace sage {

template <bool BF16, bool VEC>
__device__ __forceinline__ void load8(const uint16_t* row, int c0, int d, float v[8]) {
    if constexpr (VEC) {
        if (c0 < d) {
            uint4 raw = *reinterpret_cast<const uint4*>(row + c0);
            const uint16_t* e = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = Half<BF16>::to_f(e[j]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = 0.f;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (c0 + j < d) ? Half<BF16>::to_f(row[c0 + j]) : 0.f;
    }
}

// The 8 raw 16-bit values of channels c0 .. c0+7 of a row, zeros past d.
// The row must exist: every access stays inside it (channels past d read
// channel 0 or d - 1 and are then replaced by zeros), and there is no branch,
// so that a thread's loads of several rows are all in flight together.
template <bool VEC>
__device__ __forceinline__ uint4 load_raw8(const uint16_t* row, int c0, int d) {
    if constexpr (VEC) {
        const bool in = c0 < d;
        const uint4 r = *reinterpret_cast<const uint4*>(row + (in ? c0 : 0));
        return in ? r : make_uint4(0u, 0u, 0u, 0u);
    } else {
        uint16_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint16_t x = row[min(c0 + j, d - 1)];
            e[j] = c0 + j < d ? x : (uint16_t)0;
        }
        return make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16), e[4] | ((uint32_t)e[5] << 16),
                          e[6] | ((uint32_t)e[7] << 16));
    }
}

// load_raw8 in two halves, for a workgroup that issues other loads before it
// reads the row values: the load (channel 0 in place of channels past d) and
// the mask that zeroes those channels.  A select on the loaded value right
// after the load would make the workgroup wait for it there.
template <bool VEC>
__device__ __forceinline__ uint4 load_raw8_unmasked(const uint16_t* row, int c0, int d) {
    if constexpr (VEC) return *reinterpret_cast<const uint4*>(row + (c0 < d ? c0 : 0));
    else return load_raw8<false>(row, c0, d);
}
template <bool VEC>
__device__ __forceinline__ uint4 mask_raw8(const uint4& r, int c0, int d) {
    if constexpr (VEC) return c0 < d ? r : make_uint4(0u, 0u, 0u, 0u);
    else return r;
}

// Workgroup id -> (unit, head, sequence), the head varying fastest: with
// token-major layouts (NHD, packed varlen) the rows of all heads of a token
// are adjacent, so workgroups that run together read adjacent memory.
struct UnitHeadB {
    int unit, h, b;
};
__device__ __forceinline__ UnitHeadB unit_head_b(int bid, int units, int H) {
    return UnitHeadB{(bid / H) % units, bid % H, bid / H / units};
}

// Tokens of sequence b: [n0, n0 + N).  A varlen sequence longer than the
// maximum length the call was given (Ndense) is cut to its first Ndense
// tokens, which is all its padded slot holds.
__device__ __forceinline__ void seq_range(const int32_t* cu, int b, int Ndense, int& n0, int& N) {
    if (cu) {
        n0 = cu[b];
        N = min(max(cu[b + 1] - n0, 0), Ndense);
    } else {
        n0 = 0;
        N = Ndense;
    }
}

__device__ __forceinline__ const uint16_t* row_ptr(const void* base, int64_t sb, int64_t sh, int64_t sn,
                                                   const int32_t* cu, int b, int h, int n0, int n) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base);
    int64_t off = cu ? (int64_t)(n0 + n) * sn + (int64_t)h * sh
                     : (int64_t)b * sb + (int64_t)h * sh + (int64_t)n * sn;
    return p + off;
}

// ---------------------------------------------------------------------------
// The statistics of one channel of one (sequence, head) from its exact sum
// and (with want_minmax) its minimum and maximum: the mean
// fl32(fl64(exact sum) / N) and the FP8 V scale amax / 448 and its
// reciprocal (amax over |v - mean| if smooth, else over |v|).
template <bool BF16>
__device__ __forceinline__ void finish_stats(typename std::conditional<BF16, double, long long>::type s, float lo,
                                             float hi, int N, bool want_minmax, bool smooth, float& mean,
                                             float& scale, float& inv) {
    mean = 0.f;
    if (N > 0) {
        double s64;
        if constexpr (BF16) s64 = s;
        else s64 = (double)s * 0x1p-24;
        mean = (float)(s64 / (double)N);
    }
    scale = 0.f;
    inv = 0.f;
    if (want_minmax && N > 0) {
        // rounding is monotonic, so max_n |fl(v_n - mean)| is reached at the
        // column's max or min
        const float amax = smooth ? fmaxf(hi - mean, mean - lo) : fmaxf(hi, -lo);
        if (amax > 0.f) {
            scale = amax / 448.0f;
            inv = 448.0f / amax;
        }
    }
}

// Statistics of one kStatsChunk-token chunk of one (sequence, head): per-channel sum
// (exact, see above) and, with MINMAX (FP8 V), min and max.  fp16 minima and
// maxima are taken on the fp16 values themselves, two per instruction (exact:
// the conversion to fp32 is exact and monotonic).
template <bool BF16, int DP, bool VEC, bool MINMAX>
__device__ __forceinline__ void stats_body(const StatsArgs& a, int chunk, int h, int b,
                                           typename std::conditional<BF16, double, long long>::type* s_sum,
                                           float* s_mn, float* s_mx) {
    constexpr int TPR = DP / 8;
    constexpr int RPP = kThreads / TPR;
    constexpr int ITER = kStatsChunk / RPP;
    using Acc = typename std::conditional<BF16, double, long long>::type;
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    int n0, N;
    seq_range(a.cu, b, a.N, n0, N);
    const int tid = threadIdx.x, cg = tid % TPR, rr = tid / TPR;
    const int t_lo = chunk * a.chunk_len, t_hi = min(N, t_lo + a.chunk_len);
    double sum[8];
    float mn[8], mx[8];
    h2 mn2[4], mx2[4];
#pragma unroll
    for (int j = 0; j < 8; ++j) { sum[j] = 0.0; mn[j] = INFINITY; mx[j] = -INFINITY; }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        mn2[q] = h2{(_Float16)INFINITY, (_Float16)INFINITY};
        mx2[q] = h2{(_Float16)-INFINITY, (_Float16)-INFINITY};
    }
    // The ITER rows of a step are loaded raw first (independent loads, all in
    // flight together), then converted and summed in row order.
    for (int t0 = t_lo; t0 < t_hi; t0 += kStatsChunk) {
        uint4 raw[ITER];
#pragma unroll
        for (int it = 0; it < ITER; ++it) {             // rows past the chunk reread its last row (ignored below)
            const int n = min(t0 + it * RPP + rr, t_hi - 1);
            raw[it] = load_raw8<VEC>(row_ptr(a.x, a.sb, a.sh, a.sn, a.cu, b, h, n0, n), cg * 8, a.d);
        }
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            if (t0 + it * RPP + rr < t_hi) {
                float v[8];
                unpack8<BF16>(raw[it], v);
#pragma unroll
                for (int j = 0; j < 8; ++j) sum[j] += (double)v[j];
                if constexpr (MINMAX && BF16) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        mn[j] = fminf(mn[j], v[j]);
                        mx[j] = fmaxf(mx[j], v[j]);
                    }
                } else if constexpr (MINMAX) {
                    const uint32_t w[4] = {raw[it].x, raw[it].y, raw[it].z, raw[it].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const h2 x = __builtin_bit_cast(h2, w[q]);
                        mn2[q] = __builtin_elementwise_min(mn2[q], x);
                        mx2[q] = __builtin_elementwise_max(mx2[q], x);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);          // one row at a time: few conversions live at once
        }
    }
    if constexpr (MINMAX && !BF16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            mn[j] = (float)mn2[j >> 1][j & 1];
            mx[j] = (float)mx2[j >> 1][j & 1];
        }
    }
    // Reduce over the RPP threads that share a channel group: first the
    // threads of one wavefront (lanes 16 apart when TPR is 16), by lane
    // exchange, then the wavefronts, through LDS.  The partial sums are exact
    // (integers for fp16, exact fp64 sums for bf16), so the order is free.
    constexpr int LPW = 64 / TPR;                       // threads of a channel group per wavefront
    constexpr int NWV = kThreads / 64;
    Acc acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if constexpr (BF16) acc[j] = sum[j];
        else acc[j] = (long long)(sum[j] * 16777216.0);   // an integer below 2^53: exact
    }
#pragma unroll
    for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc[j] += __shfl_xor(acc[j], off);
            if constexpr (MINMAX) {
                mn[j] = fminf(mn[j], __shfl_xor(mn[j], off));
                mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], off));
            }
        }
    }
    static_assert(LPW * TPR == 64, "whole channel groups per wavefront");
    const int lane = tid & 63, wv = tid >> 6;
    if (lane < TPR) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            s_sum[wv * DP + cg * 8 + j] = acc[j];
            if constexpr (MINMAX) {
                s_mn[wv * DP + cg * 8 + j] = mn[j];
                s_mx[wv * DP + cg * 8 + j] = mx[j];
            }
        }
    }
    __syncthreads();
    if (tid < DP) {
        Acc s = 0;
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll
        for (int r = 0; r < NWV; ++r) {
            s += s_sum[r * DP + tid];
            if constexpr (MINMAX) {
                lo = fminf(lo, s_mn[r * DP + tid]);
                hi = fmaxf(hi, s_mx[r * DP + tid]);
            }
        }
        const int64_t o = (((int64_t)b * a.H + h) * a.chunks + chunk) * DP + tid;
        reinterpret_cast<Acc*>(a.part_sum)[o] = s;
        if constexpr (MINMAX) {
            a.part_min[o] = lo;
            a.part_max[o] = hi;
        }
    }
}

// The statistics workgroup body with min and max when the call asks for them.
// (one LDS area serves both).
template <bool BF16, int DP, bool VEC>
__device__ __forceinline__ void stats_any(const StatsArgs& a, int chunk, int h, int b) {
    using Acc = typename std::conditional<BF16, double, long long>::type;
    __shared__ Acc s_sum[kThreads / 64 * DP];
    __shared__ float s_mn[kThreads / 64 * DP], s_mx[kThreads / 64 * DP];
    if (a.want_minmax) stats_body<BF16, DP, VEC, true>(a, chunk, h, b, s_sum, s_mn, s_mx);
    else stats_body<BF16, DP, VEC, false>(a, chunk, h, b, s_sum, s_mn, s_mx);
}

// Channel statistics of one (sequence, head) for a tile workgroup: threads
// The whole workgroup reduces the (at most kMaxChunks) chunk partials of its
// (sequence, head): kThreads / DP threads per channel, each with all its
// loads in flight at once, then one exact combination per channel (integer
// sums, or fp64 sums that are exact on these inputs, so the order does not
// matter).  Tile 0 stores the caller's outputs; mean and inverse scale land
// in LDS for all threads.
template <bool BF16, int DP>
__device__ __forceinline__ void tile_stats(const StatsArgs& a, int tile, int h, int b, float* s_mu, float* s_inv) {
    using Acc = typename std::conditional<BF16, double, long long>::type;
    constexpr int TPC = kThreads / DP;                  // threads per channel
    constexpr int PER = kMaxChunks / TPC;               // chunk slots per thread
    static_assert(PER * TPC == kMaxChunks, "chunk slots");
    __shared__ Acc r_sum[kThreads];
    __shared__ float r_lo[kThreads], r_hi[kThreads];
    const int tid = threadIdx.x, c = tid % DP, part = tid / DP;
    const int64_t base = ((int64_t)b * a.H + h) * a.chunks * a.dp + c;
    Acc sum = 0;
    float lo = INFINITY, hi = -INFINITY;
    // Batches of up to 8 slots per thread: every slot of a batch loads
    // (slots past the last chunk reread chunk 0 and are ignored), so that a
    // batch's loads are in flight together; a batch runs only if some chunk
    // falls in it (a uniform branch).
    constexpr int NB = 8 < PER ? 8 : PER;
    static_assert(PER % NB == 0, "whole batches");
#pragma unroll
    for (int i0 = 0; i0 < PER; i0 += NB) {
        if (TPC * i0 >= a.chunks) break;
        Acc ps[NB];
        float pl[NB], ph[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int k = part + TPC * (i0 + i);
            const int64_t o = base + (int64_t)(k < a.chunks ? k : 0) * a.dp;
            ps[i] = reinterpret_cast<const Acc*>(a.part_sum)[o];
            if (a.want_minmax) {
                pl[i] = a.part_min[o];
                ph[i] = a.part_max[o];
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (part + TPC * (i0 + i) < a.chunks) {
                sum += ps[i];
                if (a.want_minmax) {
                    lo = fminf(lo, pl[i]);
                    hi = fmaxf(hi, ph[i]);
                }
            }
        }
    }
    r_sum[tid] = sum;
    r_lo[tid] = lo;
    r_hi[tid] = hi;
    __syncthreads();
    if (tid < DP) {
#pragma unroll
        for (int j = 1; j < TPC; ++j) {
            sum += r_sum[tid + j * DP];
            lo = fminf(lo, r_lo[tid + j * DP]);
            hi = fmaxf(hi, r_hi[tid + j * DP]);
        }
        int n0, N;
        seq_range(a.cu, b, a.N, n0, N);
        float mean, sc, iv;
        finish_stats<BF16>(sum, lo, hi, N, a.want_minmax, a.smooth, mean, sc, iv);
        const int64_t o = ((int64_t)b * a.H + h) * DP + tid;
        if (tile == 0) {
            if (a.out_mean) a.out_mean[o] = mean;
            if (a.out_scale) a.out_scale[o] = sc;
        }
        s_mu[tid] = mean;
        if (s_inv) s_inv[tid] = iv;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// INT8 quantization of one 128-row tile of Q or K.  With ks (K with
// smoothing) the workgroup subtracts the channel means, which it reduces
// from the statistics partials while its row loads are in flight.
template <bool BF16, int DP, bool VEC>
__device__ __forceinline__ void quant_rows_body(const QuantRowsArgs& a, int tile, int h, int b, const StatsArgs* ks) {
    constexpr int TPR = DP / 8;
    constexpr int RPP = kThreads / TPR;
    constexpr int PASSES = kPad / RPP;
    int n0, N;
    seq_range(a.cu, b, a.N, n0, N);
    const int tid = threadIdx.x, cg = tid % TPR, rr = tid / TPR;
    const int row0 = tile * kPad;
    // a varlen sequence's tiles past its end are never read: not written
    if (a.cu && row0 >= N) return;
    __shared__ float rmax[kPad];
    // all row loads first (rows past the sequence reread its last row), then
    // the conversion; rows past the sequence become zeros
    uint4 raw[PASSES];
    if (N > 0) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int n = min(row0 + p * RPP + rr, N - 1);
            raw[p] = load_raw8_unmasked<VEC>(row_ptr(a.x, a.sb, a.sh, a.sn, a.cu, b, h, n0, n), cg * 8, a.d);
        }
    }
    // the statistics partials are read while the rows are in flight (one
    // memory round trip instead of two)
    __shared__ float s_mu[DP];
    if (ks) tile_stats<BF16, DP>(*ks, tile, h, b, s_mu, nullptr);
    float vals[PASSES][8];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const bool in = row0 + p * RPP + rr < N;
        unpack8<BF16>(N > 0 ? mask_raw8<VEC>(raw[p], cg * 8, a.d) : make_uint4(0u, 0u, 0u, 0u), vals[p]);
#pragma unroll
        for (int j = 0; j < 8; ++j) vals[p][j] = in ? vals[p][j] : 0.f;
    }
    float mu[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) mu[j] = ks ? s_mu[cg * 8 + j] : 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = p * RPP + rr, n = row0 + r;
        float m = 0.f;
        if (n < N) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                vals[p][j] = vals[p][j] - mu[j];
                m = fmaxf(m, fabsf(vals[p][j]));
            }
        }
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (cg == 0) rmax[r] = m;
    }
    __syncthreads();
    const int G = 1 << a.group_shift;
    for (int s = 1; s < G; s <<= 1) {
        if (tid < kPad && (tid & (2 * s - 1)) == 0) rmax[tid] = fmaxf(rmax[tid], rmax[tid + s]);
        __syncthreads();
    }
    // one thread per group: the scale and its multiplier
    __shared__ float rinv[kPad];
    if (tid < kPad && (tid & (G - 1)) == 0) {
        float sc, iv;
        int8_group_scale(rmax[tid], sc, iv);
        rinv[tid] = iv;
        a.scale[((int64_t)b * a.H + h) * (a.npad >> a.group_shift) + ((row0 + tid) >> a.group_shift)] = sc;
    }
    __syncthreads();
    int8_t* obase = a.out + (((int64_t)b * a.H + h) * a.npad + row0) * DP;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = p * RPP + rr;
        *reinterpret_cast<uint2*>(obase + (int64_t)r * DP + cg * 8) = int8_codes8(vals[p], rinv[r & ~(G - 1)]);
    }
}

// Pass 1 of the Q/K quantization: workgroups [0, nq_blocks) quantize Q
// tiles; the others collect K statistics (smooth_k) or quantize K tiles.
template <bool BF16, int DP, bool VEC>
__global__ __launch_bounds__(kThreads) void qk_pass1_kernel(QuantRowsArgs q, QuantRowsArgs k, StatsArgs ks,
                                                            int nq_blocks, int smooth) {
    int bid = blockIdx.x;
    if (bid < nq_blocks) {
        const int tiles = q.npad / kPad;
        const UnitHeadB u = unit_head_b(bid, tiles, q.H);
        quant_rows_body<BF16, DP, VEC>(q, u.unit, u.h, u.b, nullptr);
        return;
    }
    bid -= nq_blocks;
    if (smooth) {
        const UnitHeadB u = unit_head_b(bid, ks.chunks, ks.H);
        stats_any<BF16, DP, VEC>(ks, u.unit, u.h, u.b);
    } else {
        const int tiles = k.npad / kPad;
        const UnitHeadB u = unit_head_b(bid, tiles, k.H);
        quant_rows_body<BF16, DP, VEC>(k, u.unit, u.h, u.b, nullptr);
    }
}

// Pass 2 (smooth_k): K tiles, minus the mean of their (sequence, head);
// tile 0 stores k_mean.
template <bool BF16, int DP, bool VEC>
__global__ __launch_bounds__(kThreads) void k_pass2_kernel(QuantRowsArgs k, StatsArgs ks) {
    const int tiles = k.npad / kPad;
    const UnitHeadB u = unit_head_b(blockIdx.x, tiles, k.H);
    quant_rows_body<BF16, DP, VEC>(k, u.unit, u.h, u.b, &ks);
}

// ---------------------------------------------------------------------------
template <bool BF16, int DP, bool VEC>
__global__ __launch_bounds__(kThreads) void v_stats_kernel(StatsArgs vs) {
    const int bid = blockIdx.x;
    const UnitHeadB u = unit_head_b(bid, vs.chunks, vs.H);
    stats_any<BF16, DP, VEC>(vs, u.unit, u.h, u.b);
}

// V -> V^T codes for one 128-key tile.  With statistics, the workgroup
// reduces the channel means / FP8 scales of its (sequence, head) while its
// loads are in flight (tile 0 stores v_scale and v_mean).
template <bool BF16, int DP, bool FP8, bool VEC>
__device__ __forceinline__ void quant_v_body(const QuantVArgs& a, const StatsArgs& vs, int have_stats, int tile,
                                             int h, int b) {
    // Thread (g, cg) loads the 8 channels cg*8 .. +7 of KPG consecutive keys
    // g*KPG .. +KPG-1 of the 128-key tile (every wavefront reads whole rows),
    // so that each channel's codes of 4 consecutive keys, which sit next to
    // each other in the permuted V^T order, leave as one LDS word.
    constexpr int TPR = DP / 8;                         // threads per key row
    constexpr int NG = kThreads / TPR;                  // key groups per tile
    constexpr int KPG = kPad / NG;                      // consecutive keys per thread (8 or 4)
    static_assert(KPG % 4 == 0, "whole 4-key groups per thread");
    constexpr int E = FP8 ? 1 : 2;                      // bytes per element
    constexpr int ROWB = kPad * E;                      // bytes per channel row of the tile in LDS
    int n0, N;
    seq_range(a.cu, b, a.N, n0, N);
    const int tid = threadIdx.x, cg = tid % TPR, g = tid / TPR;
    const int row0 = tile * kPad;
    if (a.cu && row0 >= N) return;                      // (as for the row tiles)
    __shared__ __attribute__((aligned(16))) uint8_t sv[DP * ROWB];
    const int64_t hb = ((int64_t)b * a.H + h) * DP;
    uint4 raw[KPG];
    if (N > 0) {
#pragma unroll
        for (int p = 0; p < KPG; ++p) {                 // keys past the sequence reread its last key
            const int n = min(row0 + g * KPG + p, N - 1);
            raw[p] = load_raw8_unmasked<VEC>(row_ptr(a.v, a.sb, a.sh, a.sn, a.cu, b, h, n0, n), cg * 8, a.d);
        }
    }
    // the statistics partials are read while the keys are in flight
    __shared__ float s_mu[DP], s_inv[DP];
    if (have_stats) tile_stats<BF16, DP>(vs, tile, h, b, s_mu, s_inv);
    float v[KPG][8];
#pragma unroll
    for (int p = 0; p < KPG; ++p) {
        const bool in = row0 + g * KPG + p < N;
        unpack8<BF16>(N > 0 ? mask_raw8<VEC>(raw[p], cg * 8, a.d) : make_uint4(0u, 0u, 0u, 0u), v[p]);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[p][j] = in ? v[p][j] : 0.f;
    }
    float mu[8], inv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        mu[j] = (have_stats && vs.smooth) ? s_mu[cg * 8 + j] : 0.f;
        inv[j] = (have_stats && FP8) ? s_inv[cg * 8 + j] : 1.f;
    }
    // 16-byte chunks of a channel row are XOR-swizzled by the channel group
    // so that the 16 channel groups of a wavefront hit different banks
    auto chunk_swz = [](int c) { return (c >> 3) & 7; };
#pragma unroll
    for (int q4 = 0; q4 < KPG / 4; ++q4) {
        const int kk = (g * KPG + 4 * q4);              // first of 4 consecutive keys (tile-relative)
        const int pos = (kk & ~63) | v_perm_pos(kk & 63);   // their 4 consecutive positions start here
        bool valid[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) valid[e] = row0 + kk + e < N;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = cg * 8 + j;
            const int byte = pos * E;
            uint8_t* dst = sv + c * ROWB + (((byte >> 4) ^ chunk_swz(c)) << 4) + (byte & 15);
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = v[4 * q4 + e][j] - mu[j];
            if constexpr (FP8) {
                float tq[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float tt = fminf(fmaxf(x[e] * inv[j], -448.f), 448.f);
                    tq[e] = valid[e] ? tt : 0.f;
                }
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(tq[0], tq[1], 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(tq[2], tq[3], w, true);
                *reinterpret_cast<int*>(dst) = w;
            } else {
                uint16_t hv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = valid[e] ? Half<BF16>::from_f(x[e]) : 0;
                uint2 w;
                w.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
                w.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
                *reinterpret_cast<uint2*>(dst) = w;
            }
        }
    }
    __syncthreads();
    constexpr int CPR = ROWB / 16;
    constexpr int TOTAL = DP * CPR;
    uint8_t* out = reinterpret_cast<uint8_t*>(a.vt) + (hb * a.npad + row0) * E;
    for (int L = tid; L < TOTAL; L += kThreads) {
        const int c = L / CPR, jc = L % CPR;
        *reinterpret_cast<uint4*>(out + (int64_t)c * a.npad * E + jc * 16) =
            *reinterpret_cast<const uint4*>(sv + c * ROWB + ((jc ^ chunk_swz(c)) << 4));
    }
}

template <bool BF16, int DP, bool FP8, bool VEC>
__global__ __launch_bounds__(kThreads) void quant_v_kernel(QuantVArgs a, StatsArgs vs, int have_stats) {
    const int tiles = a.npad / kPad;
    const UnitHeadB u = unit_head_b(blockIdx.x, tiles, a.H);
    quant_v_body<BF16, DP, FP8, VEC>(a, vs, have_stats, u.unit, u.h, u.b);
}

// ---------------------------------------------------------------------------
// Q, K and V in two launches (the same workgroup bodies as above).
// Pass 1: K statistics chunks (smooth_k) or K tiles; V statistics chunks
// (when V needs them); Q tiles -- in that order of workgroup ids, so that the
// statistics workgroups, whose reduction follows their loads, start first.
// Pass 2: K tiles minus their means (smooth_k); V tiles.
template <bool BF16, int DP, bool VEC>
__global__ __launch_bounds__(kThreads) void qkv_pass1_kernel(QuantRowsArgs q, QuantRowsArgs k, StatsArgs ks,
                                                             StatsArgs vs, int nq_blocks, int nk_blocks,
                                                             int smooth_k) {
    int bid = blockIdx.x;
    if (bid < nk_blocks) {
        if (smooth_k) {
            const UnitHeadB u = unit_head_b(bid, ks.chunks, ks.H);
            stats_any<BF16, DP, VEC>(ks, u.unit, u.h, u.b);
        } else {
            const int tiles = k.npad / kPad;
            const UnitHeadB u = unit_head_b(bid, tiles, k.H);
            quant_rows_body<BF16, DP, VEC>(k, u.unit, u.h, u.b, nullptr);
        }
        return;
    }
    bid -= nk_blocks;
    const int nv_blocks = (int)gridDim.x - nk_blocks - nq_blocks;
    if (bid < nv_blocks) {
        const UnitHeadB u = unit_head_b(bid, vs.chunks, vs.H);
        stats_any<BF16, DP, VEC>(vs, u.unit, u.h, u.b);
        return;
    }
    bid -= nv_blocks;
    const int tiles = q.npad / kPad;
    const UnitHeadB u = unit_head_b(bid, tiles, q.H);
    quant_rows_body<BF16, DP, VEC>(q, u.unit, u.h, u.b, nullptr);
}

template <bool BF16, int DP, bool FP8, bool VEC>
__global__ __launch_bounds__(kThreads) void qkv_pass2_kernel(QuantRowsArgs k, StatsArgs ks, QuantVArgs v,
                                                             StatsArgs vs, int nk_blocks, int v_stats) {
    int bid = blockIdx.x;
    if (bid < nk_blocks) {
        const int tiles = k.npad / kPad;
        const UnitHeadB u = unit_head_b(bid, tiles, k.H);
        quant_rows_body<BF16, DP, VEC>(k, u.unit, u.h, u.b, &ks);
        return;
    }
    bid -= nk_blocks;
    const int tiles = v.npad / kPad;
    const UnitHeadB u = unit_head_b(bid, tiles, v.H);
    quant_v_body<BF16, DP, FP8, VEC>(v, vs, v_stats, u.unit, u.h, u.b);
}

template <bool BF16, int DP, bool FP8, bool VEC>
static hipError_t quant_qkv_dispatch(const QuantRowsArgs& q, const QuantRowsArgs& k, const StatsArgs& ks,
                                     bool smooth_k, const QuantVArgs& v, const StatsArgs& vs, bool v_stats,
                                     hipStream_t s) {
    const int nq = q.out ? (q.npad / kPad) * q.H * q.B : 0;       // no Q output: K and V only
    const int k_tiles = (k.npad / kPad) * k.H * k.B;
    const int nk1 = smooth_k ? ks.chunks * ks.H * ks.B : k_tiles;
    const int nv1 = v_stats ? vs.chunks * vs.H * vs.B : 0;
    qkv_pass1_kernel<BF16, DP, VEC><<<nq + nk1 + nv1, kThreads, 0, s>>>(q, k, ks, vs, nq, nk1, smooth_k ? 1 : 0);
    if (hipError_t e = hipGetLastError()) return e;
    const int nk2 = smooth_k ? k_tiles : 0;
    const int nv2 = (v.npad / kPad) * v.H * v.B;
    qkv_pass2_kernel<BF16, DP, FP8, VEC><<<nk2 + nv2, kThreads, 0, s>>>(k, ks, v, vs, nk2, v_stats ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_quant_qkv(const QuantRowsArgs& q, const QuantRowsArgs& k, const StatsArgs& ks, bool smooth_k,
                            const QuantVArgs& v, const StatsArgs& vs, bool v_stats, bool bf16, bool fp8, bool vec,
                            hipStream_t s) {
    const int dp = q.d <= 64 ? 64 : 128;
#define SAGE_QKV(BF, D, F, V) return quant_qkv_dispatch<BF, D, F, V>(q, k, ks, smooth_k, v, vs, v_stats, s)
#define SAGE_QKV2(BF, D, F) { if (vec) SAGE_QKV(BF, D, F, true); else SAGE_QKV(BF, D, F, false); }
    if (bf16) {
        if (dp == 128) { if (fp8) SAGE_QKV2(true, 128, true) else SAGE_QKV2(true, 128, false) }
        else { if (fp8) SAGE_QKV2(true, 64, true) else SAGE_QKV2(true, 64, false) }
    } else {
        if (dp == 128) { if (fp8) SAGE_QKV2(false, 128, true) else SAGE_QKV2(false, 128, false) }
        else { if (fp8) SAGE_QKV2(false, 64, true) else SAGE_QKV2(false, 64, false) }
    }
#undef SAGE_QKV2
#undef SAGE_QKV
}

// ---------------------------------------------------------------------------
// launchers
template <bool BF16, int DP, bool VEC>
static hipError_t quant_qk_dispatch(const QuantRowsArgs& q, const QuantRowsArgs& k, const StatsArgs& ks, bool smooth,
                                    hipStream_t s) {
    const int nq = q.out ? (q.npad / kPad) * q.H * q.B : 0;       // no Q output: K only
    const int n2 = smooth ? ks.chunks * ks.H * ks.B : (k.npad / kPad) * k.H * k.B;
    qk_pass1_kernel<BF16, DP, VEC><<<nq + n2, kThreads, 0, s>>>(q, k, ks, nq, smooth ? 1 : 0);
    if (smooth) {
        if (hipError_t e = hipGetLastError()) return e;
        k_pass2_kernel<BF16, DP, VEC><<<(k.npad / kPad) * k.H * k.B, kThreads, 0, s>>>(k, ks);
    }
    return hipGetLastError();
}

hipError_t launch_quant_qk(const QuantRowsArgs& q, const QuantRowsArgs& k, const StatsArgs& ks, bool smooth,
                           bool bf16, bool vec, hipStream_t s) {
    const int dp = q.d <= 64 ? 64 : 128;
#define SAGE_QK(BF, D, V) return quant_qk_dispatch<BF, D, V>(q, k, ks, smooth, s)
    if (bf16) {
        if (dp == 128) { if (vec) SAGE_QK(true, 128, true); else SAGE_QK(true, 128, false); }
        else { if (vec) SAGE_QK(true, 64, true); else SAGE_QK(true, 64, false); }
    } else {
        if (dp == 128) { if (vec) SAGE_QK(false, 128, true); else SAGE_QK(false, 128, false); }
        else { if (vec) SAGE_QK(false, 64, true); else SAGE_QK(false, 64, false); }
    }
#undef SAGE_QK
}

template <bool BF16, int DP, bool FP8, bool VEC>
static hipError_t quant_v_dispatch(const QuantVArgs& a, const StatsArgs& vs, bool stats, bool smooth, hipStream_t s) {
    if (stats) {
        v_stats_kernel<BF16, DP, VEC><<<vs.chunks * vs.H * vs.B, kThreads, 0, s>>>(vs);
        if (hipError_t e = hipGetLastError()) return e;
    }
    quant_v_kernel<BF16, DP, FP8, VEC><<<(a.npad / kPad) * a.H * a.B, kThreads, 0, s>>>(a, vs, stats ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_quant_v(const QuantVArgs& a, const StatsArgs& vs, bool stats, bool smooth, bool bf16, bool fp8,
                          bool vec, hipStream_t s) {
    const int dp = a.d <= 64 ? 64 : 128;
#define SAGE_QV(BF, D, F, V) return quant_v_dispatch<BF, D, F, V>(a, vs, stats, smooth, s)
#define SAGE_QV2(BF, D, F) { if (vec) SAGE_QV(BF, D, F, true); else SAGE_QV(BF, D, F, false); }
    if (bf16) {
        if (dp == 128) { if (fp8) SAGE_QV2(true, 128, true) else SAGE_QV2(true, 128, false) }
        else { if (fp8) SAGE_QV2(true, 64, true) else SAGE_QV2(true, 64, false) }
    } else {
        if (dp == 128) { if (fp8) SAGE_QV2(false, 128, true) else SAGE_QV2(false, 128, false) }
        else { if (fp8) SAGE_QV2(false, 64, true) else SAGE_QV2(false, 64, false) }
    }
#undef SAGE_QV2
#undef SAGE_QV
}

}  // namespace sage
