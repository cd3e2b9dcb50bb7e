// quant.hip -- HBM-bound quantize passes for the quantized attention forward
// (gfx950).
//
//   stats_kernel     exact per-channel sums of K or V along the sequence
//                    (plus min/max for FP8 V), one workgroup per 256-token
//                    chunk of one (sequence, head);
//   finalize_kernel  chunk partials -> mean, and for FP8 V the per-channel
//                    scale amax/448 and its reciprocal;
//   quant_rows_kernel  Q or K rows -> INT8 codes + one fp32 scale per group
//                    of rows (per_block / per_warp / per_thread);
//   quant_v_kernel   V -> transposed FP8 E4M3FN codes (or fp16/bf16), keys
//                    reordered inside each 64-key block for the P.V MFMA.
//
// Method ("SageAttention deployment guide", pwwt.cn): sec. 1 first bullet
// (Q, K -> INT8 with per-block / per-thread scale factors), second bullet
// (V -> FP8), sec. 4.2 (qk_quant_gran; smooth_k subtracts K's mean along the
// sequence; smooth_v subtracts V's mean).
//
// Bit-exactness: a mean is fl32(fl64(exact sum) / N).  fp16 inputs are
// summed as int64 multiples of 2^-24 (every fp16 value is one; exact for
// N < 2^23).  bf16 inputs are summed in fp64, which is exact -- and therefore
// independent of the summation order -- when a column's values span fewer
// than 53 bits including log2(N).  The quantizer's fp32 operations are single
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

__device__ __forceinline__ void seq_range(const int32_t* cu, int b, int Ndense, int& n0, int& N) {
    if (cu) {
        n0 = cu[b];
        N = cu[b + 1] - n0;
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
template <bool BF16, int DP, bool VEC>
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsArgs a) {
    constexpr int TPR = DP / 8;
    constexpr int RPP = kThreads / TPR;
    using Acc = typename std::conditional<BF16, double, long long>::type;
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    int n0, N;
    seq_range(a.cu, b, a.N, n0, N);
    const int tid = threadIdx.x, cg = tid % TPR, rr = tid / TPR;
    const int t0 = chunk * kStatsChunk;
    Acc sum[8];
    float mn[8], mx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) { sum[j] = 0; mn[j] = INFINITY; mx[j] = -INFINITY; }
    for (int r = rr; r < kStatsChunk; r += RPP) {
        const int n = t0 + r;
        if (n >= N) break;
        float v[8];
        load8<BF16, VEC>(row_ptr(a.x, a.sb, a.sh, a.sn, a.cu, b, h, n0, n), cg * 8, a.d, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (BF16) sum[j] += (double)v[j];
            else sum[j] += (long long)(v[j] * 16777216.0f);   // exact: v * 2^24 is an integer
            mn[j] = fminf(mn[j], v[j]);
            mx[j] = fmaxf(mx[j], v[j]);
        }
    }
    // reduce over the RPP threads that share a channel group, in a fixed order
    __shared__ Acc s_sum[RPP][DP];
    __shared__ float s_mn[RPP][DP], s_mx[RPP][DP];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        s_sum[rr][cg * 8 + j] = sum[j];
        s_mn[rr][cg * 8 + j] = mn[j];
        s_mx[rr][cg * 8 + j] = mx[j];
    }
    __syncthreads();
    if (tid < DP) {
        Acc s = 0;
        float lo = INFINITY, hi = -INFINITY;
        for (int r = 0; r < RPP; ++r) {
            s += s_sum[r][tid];
            lo = fminf(lo, s_mn[r][tid]);
            hi = fmaxf(hi, s_mx[r][tid]);
        }
        const int64_t o = (((int64_t)b * a.H + h) * a.chunks + chunk) * DP + tid;
        reinterpret_cast<Acc*>(a.part_sum)[o] = s;
        if (a.want_minmax) {
            a.part_min[o] = lo;
            a.part_max[o] = hi;
        }
    }
}

template <bool BF16>
__global__ void finalize_kernel(FinalizeArgs a) {
    using Acc = typename std::conditional<BF16, double, long long>::type;
    const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
    if (c >= a.dp) return;
    int n0, N;
    seq_range(a.cu, b, a.N, n0, N);
    const int64_t base = ((int64_t)b * a.H + h) * a.chunks * a.dp + c;
    Acc s = 0;
    float lo = INFINITY, hi = -INFINITY;
    for (int k = 0; k < a.chunks; ++k) {
        s += reinterpret_cast<const Acc*>(a.part_sum)[base + (int64_t)k * a.dp];
        if (a.mode == 1) {
            lo = fminf(lo, a.part_min[base + (int64_t)k * a.dp]);
            hi = fmaxf(hi, a.part_max[base + (int64_t)k * a.dp]);
        }
    }
    float mean = 0.f;
    if (N > 0) {
        double s64;
        if constexpr (BF16) s64 = s;
        else s64 = (double)s * 0x1p-24;
        mean = (float)(s64 / (double)N);
    }
    const int64_t o = ((int64_t)b * a.H + h) * a.dp + c;
    if (a.mean) a.mean[o] = mean;
    if (a.mode == 1) {
        float amax = 0.f;
        if (N > 0) {
            // rounding is monotonic, so max_n |fl(v_n - mean)| is reached at
            // the column's max or min
            if (a.smooth) amax = fmaxf(hi - mean, mean - lo);
            else amax = fmaxf(hi, -lo);
        }
        a.v_scale[o] = amax > 0.f ? amax / 448.0f : 0.f;
        a.v_inv[o] = amax > 0.f ? 448.0f / amax : 0.f;
    }
}

// ---------------------------------------------------------------------------
template <bool BF16, int DP, bool VEC>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(QuantRowsArgs a) {
    constexpr int TPR = DP / 8;
    constexpr int RPP = kThreads / TPR;
    constexpr int PASSES = kPad / RPP;
    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    int n0, N;
    seq_range(a.cu, b, a.N, n0, N);
    const int tid = threadIdx.x, cg = tid % TPR, rr = tid / TPR;
    const int row0 = tile * kPad;
    __shared__ float rmax[kPad];
    float mu[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) mu[j] = a.mean ? a.mean[((int64_t)b * a.H + h) * DP + cg * 8 + j] : 0.f;
    float vals[PASSES][8];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = p * RPP + rr, n = row0 + r;
        float m = 0.f;
        if (n < N) {
            load8<BF16, VEC>(row_ptr(a.x, a.sb, a.sh, a.sn, a.cu, b, h, n0, n), cg * 8, a.d, vals[p]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                vals[p][j] = vals[p][j] - mu[j];
                m = fmaxf(m, fabsf(vals[p][j]));
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) vals[p][j] = 0.f;
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
    int8_t* obase = a.out + (((int64_t)b * a.H + h) * a.npad + row0) * DP;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = p * RPP + rr;
        const float amax = rmax[r & ~(G - 1)];
        const float inv = amax > 0.f ? 127.0f / amax : 0.f;
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float t = vals[p][j] * inv;
            t = __builtin_rintf(t);
            t = fminf(fmaxf(t, -127.f), 127.f);
            w[j >> 2] |= ((uint32_t)((int)t & 0xff)) << (8 * (j & 3));
        }
        *reinterpret_cast<uint2*>(obase + (int64_t)r * DP + cg * 8) = make_uint2(w[0], w[1]);
        if (cg == 0 && (r & (G - 1)) == 0)
            a.scale[((int64_t)b * a.H + h) * (a.npad >> a.group_shift) + ((row0 + r) >> a.group_shift)] =
                amax > 0.f ? amax / 127.0f : 0.f;
    }
}

// ---------------------------------------------------------------------------
template <bool BF16, int DP, bool FP8, bool VEC>
__global__ __launch_bounds__(kThreads) void quant_v_kernel(QuantVArgs a) {
    constexpr int TPR = DP / 8;
    constexpr int RPP = kThreads / TPR;
    constexpr int PASSES = kPad / RPP;
    constexpr int E = FP8 ? 1 : 2;                      // bytes per element
    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    int n0, N;
    seq_range(a.cu, b, a.N, n0, N);
    const int tid = threadIdx.x, cg = tid % TPR, rr = tid / TPR;
    const int row0 = tile * kPad;
    __shared__ __attribute__((aligned(16))) uint8_t sv[DP * kPad * E];
    const int64_t hb = ((int64_t)b * a.H + h) * DP;
    float mu[8], inv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        mu[j] = a.mean ? a.mean[hb + cg * 8 + j] : 0.f;
        inv[j] = FP8 ? a.inv[hb + cg * 8 + j] : 1.f;
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int r = p * RPP + rr, n = row0 + r;
        float v[8];
        if (n < N) {
            load8<BF16, VEC>(row_ptr(a.v, a.sb, a.sh, a.sn, a.cu, b, h, n0, n), cg * 8, a.d, v);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = 0.f;
        }
        const int pos = (r & ~63) | v_perm_pos(r & 63);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = v[j] - mu[j];
            const int c = cg * 8 + j;
            if constexpr (FP8) {
                float t = x * inv[j];
                t = fminf(fmaxf(t, -448.f), 448.f);
                const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(t, 0.f, 0, false);
                sv[c * kPad + pos] = (n < N) ? (uint8_t)(pk & 0xff) : 0;
            } else {
                reinterpret_cast<uint16_t*>(sv)[c * kPad + pos] = (n < N) ? Half<BF16>::from_f(x) : 0;
            }
        }
    }
    __syncthreads();
    constexpr int ROWB = kPad * E;                       // bytes per channel row of the tile
    constexpr int CPR = ROWB / 16;
    constexpr int TOTAL = DP * CPR;
    uint8_t* out = reinterpret_cast<uint8_t*>(a.vt) + (hb * a.npad + row0) * E;
    for (int L = tid; L < TOTAL; L += kThreads) {
        const int c = L / CPR, j = L % CPR;
        *reinterpret_cast<uint4*>(out + (int64_t)c * a.npad * E + j * 16) =
            *reinterpret_cast<const uint4*>(sv + c * ROWB + j * 16);
    }
}

// ---------------------------------------------------------------------------
// launchers
template <bool BF16>
static hipError_t stats_dispatch(const StatsArgs& a, bool vec, hipStream_t s) {
    dim3 grid(a.chunks, a.H, a.B);
    if (a.dp == 128) {
        if (vec) stats_kernel<BF16, 128, true><<<grid, kThreads, 0, s>>>(a);
        else stats_kernel<BF16, 128, false><<<grid, kThreads, 0, s>>>(a);
    } else {
        if (vec) stats_kernel<BF16, 64, true><<<grid, kThreads, 0, s>>>(a);
        else stats_kernel<BF16, 64, false><<<grid, kThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_stats(const StatsArgs& a, bool bf16, hipStream_t s) {
    // vector loads need 16-byte aligned rows
    const bool vec = (reinterpret_cast<uintptr_t>(a.x) % 16 == 0) && a.d % 8 == 0 && a.sb % 8 == 0 &&
                     a.sh % 8 == 0 && a.sn % 8 == 0;
    return bf16 ? stats_dispatch<true>(a, vec, s) : stats_dispatch<false>(a, vec, s);
}

hipError_t launch_finalize(const FinalizeArgs& a, bool bf16, hipStream_t s) {
    dim3 grid(a.H, a.B);
    if (bf16) finalize_kernel<true><<<grid, 128, 0, s>>>(a);
    else finalize_kernel<false><<<grid, 128, 0, s>>>(a);
    return hipGetLastError();
}

template <bool BF16, int DP>
static void quant_rows_dispatch(const QuantRowsArgs& a, bool vec, hipStream_t s) {
    dim3 grid(a.npad / kPad, a.H, a.B);
    if (vec) quant_rows_kernel<BF16, DP, true><<<grid, kThreads, 0, s>>>(a);
    else quant_rows_kernel<BF16, DP, false><<<grid, kThreads, 0, s>>>(a);
}

hipError_t launch_quant_rows(const QuantRowsArgs& a, bool bf16, bool vec, hipStream_t s) {
    const int dp = a.d <= 64 ? 64 : 128;
    if (bf16) {
        if (dp == 128) quant_rows_dispatch<true, 128>(a, vec, s);
        else quant_rows_dispatch<true, 64>(a, vec, s);
    } else {
        if (dp == 128) quant_rows_dispatch<false, 128>(a, vec, s);
        else quant_rows_dispatch<false, 64>(a, vec, s);
    }
    return hipGetLastError();
}

template <bool BF16, int DP, bool FP8>
static void quant_v_dispatch(const QuantVArgs& a, bool vec, hipStream_t s) {
    dim3 grid(a.npad / kPad, a.H, a.B);
    if (vec) quant_v_kernel<BF16, DP, FP8, true><<<grid, kThreads, 0, s>>>(a);
    else quant_v_kernel<BF16, DP, FP8, false><<<grid, kThreads, 0, s>>>(a);
}

hipError_t launch_quant_v(const QuantVArgs& a, bool bf16, bool fp8, bool vec, hipStream_t s) {
    const int dp = a.d <= 64 ? 64 : 128;
#define SAGE_QV(BF, D, F) quant_v_dispatch<BF, D, F>(a, vec, s)
    if (bf16) {
        if (dp == 128) { if (fp8) SAGE_QV(true, 128, true); else SAGE_QV(true, 128, false); }
        else { if (fp8) SAGE_QV(true, 64, true); else SAGE_QV(true, 64, false); }
    } else {
        if (dp == 128) { if (fp8) SAGE_QV(false, 128, true); else SAGE_QV(false, 128, false); }
        else { if (fp8) SAGE_QV(false, 64, true); else SAGE_QV(false, 64, false); }
    }
#undef SAGE_QV
    return hipGetLastError();
}

}  // namespace sage
