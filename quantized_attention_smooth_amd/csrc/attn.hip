// attn.hip -- fused quantized attention forward for gfx950 (CDNA4).
//
// Method (SageAttention pages): S = Q8 K8^T as 8-bit integer products with
// int32 accumulation, dequantized by the Q and K scale factors ("SageAttention
// deployment guide", pwwt.cn, sec. 1 first bullet); softmax computed online,
// block by block, as in FlashAttention ("SageAttention 2.2.0 on the RX 9070
// XT", pnsm.cn, sec. 2); P.V with V in FP8 (or FP16/BF16) and fp32
// accumulation, output FP16/BF16 (deployment guide, sec. 1 second and third
// bullets; sec. 4.2 pv_accum_dtype); is_causal / sm_scale / return_lse as in
// the deployment guide's sec. 4.1.
//
// Mapping onto CDNA4:
//  * workgroup = 4 wavefronts = 128 query rows; wavefront w owns rows
//    32w..32w+31.  Its Q^T fragments (INT8) stay in VGPRs for the whole key
//    loop.
//  * per 64-key step the K tile (INT8, 64 x Dp) and the V^T tile (FP8 Dp x 64
//    or fp16 Dp x 64) are staged once in LDS (XOR-swizzled, double-buffered)
//    and shared by the 4 wavefronts.
//  * S^T = K Q^T with v_mfma_i32_32x32x32_i8: each lane owns one query column
//    and 16 keys per 32-key block.  The accumulators start at the bit pattern
//    of 1.5*2^23 so the result reads directly as the float 1.5*2^23 + S.
//  * the row maximum is an integer max per key-scale group, one fp32 multiply
//    per group, and one cross-half max (v_permlane32_swap); each score is then
//    one FMA and one v_exp_f32 (log2 domain, P's FP8 scale folded into the
//    exponent), and two scores become FP8 with one v_cvt_pk_fp8_f32.
//  * the lane's 32 FP8 P values are exactly the B operand of
//    v_mfma_f32_32x32x64_f8f6f4 (O^T = V^T P^T) because V^T is stored with its
//    keys in the lane order of the score accumulator.  FP16/BF16 V uses
//    v_mfma_f32_32x32x16_{f16,bf16} the same way.
//  * O^T (fp32) is rescaled only when some row of the wavefront raised its
//    running maximum.
#include "sage_device.h"

namespace sage {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2 of the FP8 P scale (448)
constexpr float kFltMin = 1.17549435e-38f;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int DP, int PV>
struct AttnCfg {
    static constexpr int NCB = DP / 32;                 // 32-channel blocks
    static constexpr int KT_BYTES = kBK * DP;           // K tile: 64 keys x Dp int8
    static constexpr int VE = PV == 0 ? 1 : 2;          // V element bytes
    static constexpr int VROW = kBK * VE;               // V^T tile row (one channel) bytes
    static constexpr int VT_BYTES = DP * VROW;
    static constexpr int STAGE = KT_BYTES + VT_BYTES;
    static constexpr int K_LOADS = KT_BYTES / (16 * kThreads);   // 16-byte loads per thread
    static constexpr int V_LOADS = VT_BYTES / (16 * kThreads);
};

// global -> registers for one key tile (K rows contiguous; V^T rows strided)
template <int DP, int PV>
__device__ __forceinline__ void load_tile(const int8_t* kbase, const uint8_t* vbase, int64_t vrow_stride,
                                          int t, int tid, uint4* kr, uint4* vr) {
    using C = AttnCfg<DP, PV>;
    const uint4* ksrc = reinterpret_cast<const uint4*>(kbase + (int64_t)t * C::KT_BYTES);
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) kr[i] = ksrc[i * kThreads + tid];
    constexpr int CPR = C::VROW / 16;
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i) {
        const int L = i * kThreads + tid, row = L / CPR, ch = L % CPR;
        vr[i] = *reinterpret_cast<const uint4*>(vbase + row * vrow_stride + (int64_t)t * C::VROW + ch * 16);
    }
}

template <int DP>
__device__ __forceinline__ void store_k(uint8_t* stage, int tid, const uint4* kr) {
    constexpr int KCPR = DP / 16;
    constexpr int K_LOADS = kBK * DP / (16 * kThreads);
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
        const int L = i * kThreads + tid, row = L / KCPR, ch = L % KCPR;
        *reinterpret_cast<uint4*>(stage + row * DP + swz<DP>(row, ch) * 16) = kr[i];
    }
}

template <int DP, int PV>
__device__ __forceinline__ void store_tile(uint8_t* stage, int tid, const uint4* kr, const uint4* vr) {
    using C = AttnCfg<DP, PV>;
    store_k<DP>(stage, tid, kr);
    constexpr int VCPR = C::VROW / 16;
    uint8_t* vs = stage + C::KT_BYTES;
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i) {
        const int L = i * kThreads + tid, row = L / VCPR, ch = L % VCPR;
        *reinterpret_cast<uint4*>(vs + row * C::VROW + swz<C::VROW>(row, ch) * 16) = vr[i];
    }
}

// S^T (64 keys x 32 queries) for one wavefront from the staged K tile.
// acc[kb][i] = bias + S(query n, key 32*kb + 8*(i/4) + 4*hh + i%4).
template <int DP>
__device__ __forceinline__ void qk_tile(const uint8_t* ks, const v4i* qf, int n, int hh, v16i acc[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        v16i c;
#pragma unroll
        for (int i = 0; i < 16; ++i) c[i] = kAccBiasBits;
        const int row = kb * 32 + n;
#pragma unroll
        for (int cb = 0; cb < DP / 32; ++cb) {
            const int ch = cb * 2 + hh;
            const v4i av = *reinterpret_cast<const v4i*>(ks + row * DP + swz<DP>(row, ch) * 16);
            c = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, qf[cb], c, 0, 0, 0);
        }
        acc[kb] = c;
    }
}

template <int DP, int PV, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnArgs a) {
    using C = AttnCfg<DP, PV>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;

    // ---- work item
    const int wg = xcd_remap(blockIdx.x, a.num_wg);
    int qt = wg % a.n_qtiles;
    const int bh = wg / a.n_qtiles, h = bh % a.Hq, b = bh / a.Hq;
    if (a.causal) qt = a.n_qtiles - 1 - qt;             // longest rows first
    int Lq = a.Nq, Lk = a.Nk, qoff = 0;
    if (a.cu_q) {
        qoff = a.cu_q[b];
        Lq = a.cu_q[b + 1] - qoff;
        Lk = a.cu_k[b + 1] - a.cu_k[b];
    }
    const int q0 = qt * kBQ;
    if (q0 >= Lq) return;                               // whole workgroup, before any barrier
    const int hk = h / (a.Hq / a.Hkv);
    const int kend = a.causal ? min(Lk, q0 + kBQ) : Lk;
    const int ntiles = (kend + kBK - 1) / kBK;

    // ---- per-lane query state
    const int qrow = q0 + wave * 32 + n;                // this lane's query row
    const int64_t qhead = (int64_t)b * a.Hq + h;
    const int8_t* q8row = a.q8 + (qhead * a.nq_pad + qrow) * DP;
    v4i qf[DP / 32];
#pragma unroll
    for (int cb = 0; cb < DP / 32; ++cb) qf[cb] = *reinterpret_cast<const v4i*>(q8row + cb * 32 + hh * 16);
    const float qscale = a.qs[qhead * (a.nq_pad >> a.gq_shift) + (qrow >> a.gq_shift)];
    const float cq = (qscale * a.sm_scale) * kLog2e;    // log2-domain factor of this row

    const int64_t khead = (int64_t)b * a.Hkv + hk;
    const int8_t* kbase = a.k8 + khead * a.nk_pad * DP;
    const float* ksbase = a.ks + khead * (a.nk_pad >> a.gk_shift);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vt) + khead * DP * a.nk_pad * C::VE;
    const int64_t vrow_stride = (int64_t)a.nk_pad * C::VE;

    v16f o[C::NCB];
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cb][i] = 0.f;
    float m_ref = -INFINITY, lsum = 0.f;
    constexpr float p_log2_scale = PV == 0 ? kLog2_448 : 0.f;

    // ---- prologue: tile 0 -> LDS buffer 0
    uint4 kr[C::K_LOADS], vr[C::V_LOADS];
    if (ntiles > 0) {
        load_tile<DP, PV>(kbase, vbase, vrow_stride, 0, tid, kr, vr);
        store_tile<DP, PV>(smem, tid, kr, vr);
    }
    __syncthreads();

    const int wave_q_lo = q0 + wave * 32;               // smallest query row of this wavefront
    for (int t = 0; t < ntiles; ++t) {
        const uint8_t* stage = smem + (t & 1) * C::STAGE;
        // prefetch the next tile (the last step reloads its own tile into the
        // idle buffer, which keeps the prefetch registers unconditional)
        load_tile<DP, PV>(kbase, vbase, vrow_stride, min(t + 1, ntiles - 1), tid, kr, vr);
        const int k0 = t * kBK;
        const bool wave_active = !a.causal || k0 <= wave_q_lo + 31;
        if (wave_active) {
            v16i acc[2];
            qk_tile<DP>(stage, qf, n, hh, acc);

            // mask keys past the sequence end and (causal) after the row
            const bool need_mask = (k0 + kBK > Lk) || (a.causal && k0 + kBK - 1 > wave_q_lo);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
                        const bool vis = key < Lk && (!a.causal || key <= qrow);
                        if (!vis) acc[kb][i] = kNegInfBits;
                    }
            }
            // key-scale group g = 2*kb + i/8 covers keys k0 + 16g .. k0 + 16g + 15
            float f[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float ksg = ksbase[(k0 + 16 * g) >> a.gk_shift];
                f[g] = fmaxf(ksg * cq, kFltMin);        // > 0, so -inf * f stays -inf
            }
            float smax = -INFINITY;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int kb = g >> 1, i0 = (g & 1) * 8;
                int mi = acc[kb][i0];
#pragma unroll
                for (int i = 1; i < 8; ++i) mi = max(mi, acc[kb][i0 + i]);
                smax = fmaxf(smax, (bits_f(mi) - kAccBias) * f[g]);
            }
            smax = swap_half_max(smax);
            float alpha = 1.f;
            const bool raise = smax > m_ref;
            if (raise) {
                alpha = __builtin_amdgcn_exp2f(m_ref - smax);   // 0 for the first visible tile
                m_ref = smax;
            }
            if (__any(raise)) {
                lsum *= alpha;
#pragma unroll
                for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
            }
            // ---- P = 2^(s - m) (times 448 on the FP8 path).  The exponent is
            // fl32(S * f + fl32(L - m)) with a single rounding: S is recovered
            // exactly from the biased accumulator (both terms lie in
            // [2^23, 2^24)), so the only inexact step after it is the FMA.
            const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
            const float nb = p_log2_scale - m_use;
            float p[2][16];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int g = 2 * kb + (i >> 3);
                    const float sf = bits_f(acc[kb][i]) - kAccBias;
                    p[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sf, f[g], nb));
                    lsum += p[kb][i];
                }
            const uint8_t* vs = stage + C::KT_BYTES;
            if constexpr (PV == 0) {
                v8i pb;
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    const int kb = w >> 2, i0 = (w & 3) * 4;
                    int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][i0], p[kb][i0 + 1], 0, false);
                    word = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][i0 + 2], p[kb][i0 + 3], word, true);
                    pb[w] = word;
                }
#pragma unroll
                for (int cb = 0; cb < C::NCB; ++cb) {
                    const int row = cb * 32 + n;
                    const v4i lo = *reinterpret_cast<const v4i*>(vs + row * C::VROW + swz<C::VROW>(row, 2 * hh) * 16);
                    const v4i hi = *reinterpret_cast<const v4i*>(vs + row * C::VROW + swz<C::VROW>(row, 2 * hh + 1) * 16);
                    const v8i va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, o[cb], 0, 0, 0, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int kb = u >> 1, i0 = (u & 1) * 8;
                    if constexpr (PV == 1) {
                        v8h pu;
#pragma unroll
                        for (int j = 0; j < 8; ++j) pu[j] = (_Float16)p[kb][i0 + j];
#pragma unroll
                        for (int cb = 0; cb < C::NCB; ++cb) {
                            const int row = cb * 32 + n;
                            const v8h va = *reinterpret_cast<const v8h*>(vs + row * C::VROW + swz<C::VROW>(row, 4 * hh + u) * 16);
                            o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pu, o[cb], 0, 0, 0);
                        }
                    } else {
                        v8bf pu;
#pragma unroll
                        for (int j = 0; j < 8; ++j) pu[j] = (__bf16)p[kb][i0 + j];
#pragma unroll
                        for (int cb = 0; cb < C::NCB; ++cb) {
                            const int row = cb * 32 + n;
                            const v8bf va = *reinterpret_cast<const v8bf*>(vs + row * C::VROW + swz<C::VROW>(row, 4 * hh + u) * 16);
                            o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pu, o[cb], 0, 0, 0);
                        }
                    }
                }
            }
        }
        store_tile<DP, PV>(smem + ((t + 1) & 1) * C::STAGE, tid, kr, vr);
        __syncthreads();
    }

    // ---- epilogue: normalise, add back V's mean, write in the caller's layout
    const float l_tot = swap_half_sum(lsum);
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float* vsc = PV == 0 ? a.vs + khead * DP : nullptr;
    const float* vmu = a.vmean ? a.vmean + khead * DP : nullptr;
    if (qrow < Lq) {
        uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) +
                         (a.cu_q ? (int64_t)(qoff + qrow) * a.on + (int64_t)h * a.oh
                                 : (int64_t)b * a.ob + (int64_t)h * a.oh + (int64_t)qrow * a.on);
#pragma unroll
        for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int c0 = cb * 32 + 8 * r4 + 4 * hh;
                if (c0 >= a.d) continue;
                uint16_t hv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = c0 + e;
                    float val = o[cb][4 * r4 + e];
                    if constexpr (PV == 0) val *= vsc[c] * inv_l;
                    else val *= inv_l;
                    if (vmu) val += vmu[c];
                    hv[e] = Half<OUT_BF16>::from_f(val);
                }
                if (a.out_vec4 && c0 + 3 < a.d) {
                    uint2 w;
                    w.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
                    w.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
                    *reinterpret_cast<uint2*>(orow + c0) = w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c0 + e < a.d) orow[c0 + e] = hv[e];
                }
            }
    }
    if (a.lse) {
        float part = 0.f;
        if (a.kmean) {
            const float* km = a.kmean + khead * DP;
#pragma unroll
            for (int cb = 0; cb < DP / 32; ++cb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int code = (int)(int8_t)((qf[cb][j >> 2] >> (8 * (j & 3))) & 0xff);
                    part += (float)code * km[cb * 32 + hh * 16 + j];
                }
        }
        const float dot = swap_half_sum(part);
        if (hh == 0 && qrow < Lq) {
            const float corr = a.kmean ? a.sm_scale * qscale * dot : 0.f;
            const float lse = (m_ref + __log2f(l_tot) - p_log2_scale) * kLn2 + corr;
            const int64_t li = a.lse_varlen ? (int64_t)h * a.total_q + qoff + qrow : qhead * a.Nq + qrow;
            a.lse[li] = lse;
        }
    }
}

// ---------------------------------------------------------------------------
// Exact int32 scores from the same K staging and QK^T tile code, for tests.
template <int DP>
__global__ __launch_bounds__(kThreads) void qk_scores_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t ks[kBK * DP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int qt = blockIdx.x % a.n_qtiles, bh = blockIdx.x / a.n_qtiles, h = bh % a.Hq, b = bh / a.Hq;
    const int hk = h / (a.Hq / a.Hkv);
    const int qrow = qt * kBQ + wave * 32 + n;
    const int64_t qhead = (int64_t)b * a.Hq + h;
    const int8_t* q8row = a.q8 + (qhead * a.nq_pad + qrow) * DP;
    v4i qf[DP / 32];
#pragma unroll
    for (int cb = 0; cb < DP / 32; ++cb) qf[cb] = *reinterpret_cast<const v4i*>(q8row + cb * 32 + hh * 16);
    const int8_t* kbase = a.k8 + ((int64_t)b * a.Hkv + hk) * a.nk_pad * DP;
    const int ntiles = (a.Nk + kBK - 1) / kBK;
    unsigned long long s1 = 0, s2 = 0;
    for (int t = 0; t < ntiles; ++t) {
        uint4 kr[kBK * DP / (16 * kThreads)];
        const uint4* ksrc = reinterpret_cast<const uint4*>(kbase + (int64_t)t * kBK * DP);
#pragma unroll
        for (int i = 0; i < kBK * DP / (16 * kThreads); ++i) kr[i] = ksrc[i * kThreads + tid];
        __syncthreads();
        store_k<DP>(ks, tid, kr);
        __syncthreads();
        v16i acc[2];
        qk_tile<DP>(ks, qf, n, hh, acc);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = t * kBK + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
                const int S = acc[kb][i] - kAccBiasBits;
                if (key < a.Nk) {
                    if (a.dbg_mode == 0) {
                        if (qrow < a.Nq)
                            reinterpret_cast<int32_t*>(a.dbg)[(qhead * a.Nq + qrow) * a.Nk + key] = S;
                    } else {
                        s1 += (unsigned long long)(long long)S;
                        s2 += (unsigned long long)(key + 1) * (unsigned long long)(long long)S;
                    }
                }
            }
    }
    if (a.dbg_mode == 1) {
        s1 += __shfl_xor(s1, 32);
        s2 += __shfl_xor(s2, 32);
        if (hh == 0 && qrow < a.Nq) {
            unsigned long long* d = reinterpret_cast<unsigned long long*>(a.dbg) + (qhead * a.Nq + qrow) * 2;
            d[0] = s1;
            d[1] = s2;
        }
    }
}

// ---------------------------------------------------------------------------
template <int DP, int PV>
static void attn_dispatch_out(const AttnArgs& a, bool out_bf16, hipStream_t s) {
    if (out_bf16) attn_fwd_kernel<DP, PV, true><<<a.num_wg, kThreads, 0, s>>>(a);
    else attn_fwd_kernel<DP, PV, false><<<a.num_wg, kThreads, 0, s>>>(a);
}

hipError_t launch_attn(const AttnArgs& a, int dp, int pv, bool out_bf16, hipStream_t s) {
    if (dp == 128) {
        if (pv == 0) attn_dispatch_out<128, 0>(a, out_bf16, s);
        else if (pv == 1) attn_dispatch_out<128, 1>(a, out_bf16, s);
        else attn_dispatch_out<128, 2>(a, out_bf16, s);
    } else {
        if (pv == 0) attn_dispatch_out<64, 0>(a, out_bf16, s);
        else if (pv == 1) attn_dispatch_out<64, 1>(a, out_bf16, s);
        else attn_dispatch_out<64, 2>(a, out_bf16, s);
    }
    return hipGetLastError();
}

hipError_t launch_qk_scores(const AttnArgs& a, int dp, hipStream_t s) {
    if (dp == 128) qk_scores_kernel<128><<<a.num_wg, kThreads, 0, s>>>(a);
    else qk_scores_kernel<64><<<a.num_wg, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sage
