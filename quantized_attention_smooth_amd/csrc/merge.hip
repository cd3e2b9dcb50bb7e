// merge.hip -- combine attention results computed over disjoint key sets.
//
// The forward can return, per query row, the natural log-sum-exp of its
// scores ("SageAttention deployment guide", pwwt.cn, sec. 4.1: return_lse,
// for Ring-Attention-style use).  When the keys of one attention are split
// into S disjoint sets and each set gives a normalised output o_s with
// log-sum-exp L_s, the attention over all keys is the convex combination
//     out = sum_s exp(L_s - L) o_s,   L = log sum_s exp(L_s),
// because exp(L_s) is the softmax denominator of set s.  This file computes
// that combination, row by row.
//
// In fp32, per row: m = max_s L_s; w_s = exp(L_s - m) (0 for L_s = -inf);
// W = sum_s w_s (s ascending); out = fl_out(sum_s (w_s / W) * o_s) with the
// sum taken s ascending; L = m + log(W).  A row whose parts are all -inf (it
// saw no key) gives out = 0 and L = -inf.
//
// The kernel is bound by HBM bandwidth: it reads S rows of d elements and S
// fp32 values per row and writes one row (and one value).  The parts are in
// the output dtype, or in fp32 when they are the split-KV forward's partial
// results (then no rounding happens before the final one).  With d a multiple
// of 8 and 16-byte aligned rows, each thread moves 8 channels (16 bytes) per
// part; consecutive threads cover consecutive 16-byte pieces of a row, then
// the next row, so every wavefront reads contiguous memory.
#include <type_traits>

#include "sage_device.h"

namespace sage {

namespace {

constexpr int kMergeThreads = 256;

struct RowWeights {
    float m, w, inv_w;
    bool empty;
};

// Reference point and normaliser of one row (every thread of the row computes
// them from the same S values, so all agree bit for bit).
__device__ __forceinline__ RowWeights row_weights(const float* lse_parts, int64_t row, int64_t rows, int S) {
    float m = -INFINITY;
    for (int s = 0; s < S; ++s) m = fmaxf(m, lse_parts[s * rows + row]);
    RowWeights r;
    r.m = m;
    r.empty = m == -INFINITY;
    float w = 0.f;
    if (!r.empty)
        for (int s = 0; s < S; ++s) w += __expf(lse_parts[s * rows + row] - m);
    r.w = w;
    r.inv_w = r.empty ? 0.f : 1.f / w;
    return r;
}

// C channels of one part row as fp32: parts stored in the output dtype
// (16-bit) or in fp32 (PF32: the split-KV forward's partial results).
template <bool BF16, bool VEC, bool PF32>
struct PartRow {
    static constexpr int C = VEC ? 8 : 1;
    typename std::conditional<PF32, float4, uint4>::type raw[(PF32 && VEC) ? 2 : 1];
    __device__ __forceinline__ void load(const void* base, int64_t off) {
        if constexpr (PF32) {
            const float* src = static_cast<const float*>(base) + off;
            if constexpr (VEC) {
                raw[0] = reinterpret_cast<const float4*>(src)[0];
                raw[1] = reinterpret_cast<const float4*>(src)[1];
            } else {
                raw[0].x = src[0];
            }
        } else {
            const uint16_t* src = static_cast<const uint16_t*>(base) + off;
            if constexpr (VEC) raw[0] = *reinterpret_cast<const uint4*>(src);
            else raw[0].x = src[0];
        }
    }
    __device__ __forceinline__ float get(int e) const {
        if constexpr (PF32) {
            if constexpr (VEC) {
                const float4& r = raw[e >> 2];
                const int k = e & 3;
                return k == 0 ? r.x : k == 1 ? r.y : k == 2 ? r.z : r.w;
            } else {
                return raw[0].x;
            }
        } else {
            if constexpr (VEC) {
                const uint32_t wds[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
                return Half<BF16>::to_f((uint16_t)(wds[e >> 1] >> (16 * (e & 1))));
            } else {
                return Half<BF16>::to_f((uint16_t)raw[0].x);
            }
        }
    }
};

template <bool BF16, bool VEC, bool PF32>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
    constexpr int C = VEC ? 8 : 1;                      // channels per thread
    const int per_row = (a.d + C - 1) / C;
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    const int64_t idx = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
    if (idx >= rows * per_row) return;
    const int64_t row = idx / per_row;
    const int c0 = (int)(idx - row * per_row) * C;
    const int64_t n = row % a.N, bh = row / a.N;
    const int64_t h = bh % a.H, b = bh / a.H;

    const RowWeights rw = row_weights(a.lse_parts, row, rows, a.S);
    const int64_t part0 = b * a.pb + h * a.ph + n * a.pn + c0;
    float acc[C];
#pragma unroll
    for (int e = 0; e < C; ++e) acc[e] = 0.f;
    // parts in groups of U: the U loads of a group are issued before any of
    // them is used, so each thread keeps U * 16 (fp32: 32) bytes in flight
    constexpr int U = 4;
    for (int s0 = 0; s0 < a.S; s0 += U) {
        PartRow<BF16, VEC, PF32> v[U];
        float ws[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u;
            if (s < a.S) {
                v[u].load(a.parts, part0 + s * a.ps);
                const float ls = a.lse_parts[s * rows + row];
                // a part that saw no key (and a row that saw none) adds nothing
                ws[u] = (rw.empty || ls == -INFINITY) ? 0.f : __expf(ls - rw.m) * rw.inv_w;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s0 + u >= a.S || ws[u] == 0.f) continue;
#pragma unroll
            for (int e = 0; e < C; ++e) acc[e] = __builtin_fmaf(ws[u], v[u].get(e), acc[e]);
        }
    }
    uint16_t* dst = static_cast<uint16_t*>(a.out) + b * a.ob + h * a.oh + n * a.on + c0;
    if constexpr (VEC) {
        uint16_t hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = Half<BF16>::from_f(acc[e]);
        uint4 o;
        o.x = hv[0] | ((uint32_t)hv[1] << 16);
        o.y = hv[2] | ((uint32_t)hv[3] << 16);
        o.z = hv[4] | ((uint32_t)hv[5] << 16);
        o.w = hv[6] | ((uint32_t)hv[7] << 16);
        *reinterpret_cast<uint4*>(dst) = o;
    } else {
        dst[0] = Half<BF16>::from_f(acc[0]);
    }
    if (a.lse && c0 == 0) a.lse[row] = rw.empty ? -INFINITY : rw.m + __logf(rw.w);
}

}  // namespace

template <bool BF16, bool VEC>
void launch_merge_parts(const MergeArgs& a, dim3 grid, dim3 block, hipStream_t s) {
    if (a.parts_f32) hipLaunchKernelGGL((merge_kernel<BF16, VEC, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<BF16, VEC, false>), grid, block, 0, s, a);
}

hipError_t launch_merge(const MergeArgs& a, bool bf16, bool vec, hipStream_t s) {
    const int C = vec ? 8 : 1;
    const int64_t threads = (int64_t)a.B * a.H * a.N * ((a.d + C - 1) / C);
    const dim3 grid((unsigned)((threads + kMergeThreads - 1) / kMergeThreads)), block(kMergeThreads);
    if (bf16) {
        if (vec) launch_merge_parts<true, true>(a, grid, block, s);
        else launch_merge_parts<true, false>(a, grid, block, s);
    } else {
        if (vec) launch_merge_parts<false, true>(a, grid, block, s);
        else launch_merge_parts<false, false>(a, grid, block, s);
    }
    return hipGetLastError();
}

}  // namespace sage
