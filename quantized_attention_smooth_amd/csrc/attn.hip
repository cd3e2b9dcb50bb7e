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
//  * workgroup = 4 wavefronts = 256 query rows, one workgroup per CU; each
//    wavefront owns 64 rows as two 32-row MFMA column blocks, whose Q^T
//    fragments (INT8) stay in VGPRs for the whole key loop.
//  * per 64-key step the K tile (INT8, 64 x Dp) and the V^T tile (FP8 Dp x 64
//    or fp16 Dp x 64) are copied global -> LDS by the DMA path
//    (global_load_lds) into a ring of NST stages, AHEAD tiles ahead, shared by
//    the 4 wavefronts; rows are XOR-swizzled so the fragment reads are free of
//    bank conflicts.
//  * S^T = K Q^T with v_mfma_i32_32x32x32_i8: each lane owns one query column
//    and 16 keys per 32-key block.  The accumulators start at the bit pattern
//    of 1.5*2^23 so the result reads directly as the float 1.5*2^23 + S.
//  * the tile maximum is an integer max per key-scale group, one fp32
//    multiply per group, and one cross-half max (v_permlane32_swap); each
//    score is then one FMA and one v_exp_f32 (log2 domain, P's FP8 scale
//    folded into the exponent), and two scores become FP8 with one
//    v_cvt_pk_fp8_f32.
//  * the lane's 32 FP8 P values are exactly the B operand of
//    v_mfma_f32_32x32x64_f8f6f4 (O^T = V^T P^T) because V^T is stored with its
//    keys in the lane order of the score accumulator.  FP16/BF16 V uses
//    v_mfma_f32_32x32x16_{f16,bf16} the same way.  The row sums of P come
//    from one more small MFMA per tile.
//  * software pipeline: while the VALU runs the softmax of tile t, the matrix
//    cores run QK^T of tile t+1 and P.V of tile t-1; the scheduler is told to
//    interleave the two streams instruction by instruction, which is what
//    lets one wavefront keep the MFMA pipe and the VALU busy together.
//  * O^T (fp32) is rescaled only when some row of the wavefront raised its
//    running maximum (lazy rescaling with threshold kTau).
#include "sage_device.h"

namespace sage {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2 of the FP8 P scale (448)
// Lazy rescaling: a row's reference maximum only moves when a tile's maximum
// exceeds it by more than kTau (log2 units), so P can reach 2^kTau and its
// FP8 scale is 448 / 2^kTau.  Most tiles then skip the O rescale.
constexpr int kTau = 3;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int DP, int PV>
struct AttnCfg {
    static constexpr int NCB = DP / 32;                 // 32-channel blocks
    static constexpr int KT_BYTES = kBK * DP;           // K tile: 64 keys x Dp int8
    static constexpr int VE = PV == 0 ? 1 : 2;          // V element bytes
    static constexpr int VROW = kBK * VE;               // V^T tile row (one channel) bytes
    static constexpr int VT_BYTES = DP * VROW;
    static constexpr int SC_OFF = KT_BYTES + VT_BYTES;  // the tile's K scales, one 16-byte slot per wavefront
    static constexpr int STAGE = KT_BYTES + VT_BYTES + 64;
    static constexpr int NI = (KT_BYTES + VT_BYTES) / (16 * kThreads);   // 1 KB DMA instructions per wavefront
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// Direct global -> LDS copy of one key tile into one stage of the ring.
// Instruction i of wavefront w fills the 1 KB of granules [(4i + w) * 64, +64);
// lane L writes granule (4i + w) * 64 + L.  The granule at (row, physical
// chunk c) receives logical chunk swz(row, c) (the swizzle is an involution),
// so readers address logical chunk c at swz(row, c).  Lanes 0-3 of every
// wavefront then copy the tile's K scales (4 groups of 16 keys, or the one
// group of 64 four times) into the wavefront's own 16-byte slot, so that the
// softmax reads them from LDS instead of issuing global loads behind the
// in-flight copies.  Every wavefront issues NI + 1 copies per tile.
template <int DP, int PV>
__device__ __forceinline__ void dma_tile(uint8_t* stage, const int8_t* kbase, const uint8_t* vbase,
                                         int64_t vrow_stride, const float* ksbase, bool ks16, int t, int wave,
                                         int lane) {
    using C = AttnCfg<DP, PV>;
    constexpr int KG = C::KT_BYTES / 16, KCPR = DP / 16, VCPR = C::VROW / 16;
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
        const int gbase = (4 * i + wave) * 64;           // wave-uniform
        const int g = gbase + lane;
        const uint8_t* src;
        if (gbase < KG) {
            const int row = g / KCPR, ch = swz<DP>(row, g % KCPR);
            src = reinterpret_cast<const uint8_t*>(kbase) + (int64_t)t * C::KT_BYTES + row * DP + ch * 16;
        } else {
            const int gv = g - KG, row = gv / VCPR, ch = swz<C::VROW>(row, gv % VCPR);
            src = vbase + row * vrow_stride + (int64_t)t * C::VROW + ch * 16;
        }
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(stage + gbase * 16), 16, 0, 0);
    }
    if (lane < 4) {
        const float* src = ks16 ? ksbase + 4 * t + lane : ksbase + t;
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(stage + C::SC_OFF + wave * 16), 4, 0, 0);
    }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that also keeps the compiler from moving LDS accesses
// across it (the hardware ordering comes from the explicit vmcnt waits).
__device__ __forceinline__ void block_sync() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Row sums of P with one small MFMA: the lane's P values are the B operand of
// a 16x16xK MFMA whose K blocks come from the four 16-lane groups.  Groups 0/2
// hold queries 0..15 (lane halves 0/1), groups 1/3 queries 16..31, so an A
// operand of ones on the rows and K blocks of matching parity gives every lane
// the sum over all 64 keys of its own query (the four values of the lane's C
// registers are equal).
__device__ __forceinline__ bool rowsum_parity(int lane) {
    return (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1);
}

// ---------------------------------------------------------------------------
// Pieces of the key loop for one wavefront (64 query rows = blocks j = 0, 1).

// K fragments of one staged tile: kf[kb][cb] is the A operand for keys
// 32*kb .. 32*kb+31 (row n of the block), channels 32*cb + 16*hh .. +15.
template <int DP>
__device__ __forceinline__ void load_kfrag(const uint8_t* ks, int n, int hh, v4i (&kf)[2][DP / 32]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int row = kb * 32 + n;
#pragma unroll
        for (int cb = 0; cb < DP / 32; ++cb)
            kf[kb][cb] = *reinterpret_cast<const v4i*>(ks + row * DP + swz<DP>(row, cb * 2 + hh) * 16);
    }
}

// S^T of one row block: S[kb][i] = bias + S(query n of the block,
// key 32*kb + 8*(i/4) + 4*hh + i%4).  Two accumulation chains over the
// channel blocks; the first MFMA of each takes the bias vector as input.
template <int DP>
__device__ __forceinline__ void qk_half(const v4i (&kf)[2][DP / 32], const v4i (&qf)[DP / 32], const v16i& biasv,
                                        v16i (&S)[2]) {
#pragma unroll
    for (int cb = 0; cb < DP / 32; ++cb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            S[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kb][cb], qf[cb], cb == 0 ? biasv : S[kb], 0, 0, 0);
}

// V^T fragments of one tile (A operand of P.V: channel row cb*32 + n, the keys
// of lane half hh).
template <int DP, int PV>
struct VFrag {
    // FP8: 32 bytes per 32-channel block; fp16/bf16: 4 x 16 bytes per block
    v4i f[DP / 32][PV == 0 ? 2 : 4];
};

template <int DP, int PV>
__device__ __forceinline__ void load_vfrag(const uint8_t* vs, int n, int hh, VFrag<DP, PV>& vf) {
    using C = AttnCfg<DP, PV>;
#pragma unroll
    for (int cb = 0; cb < DP / 32; ++cb) {
        const int row = cb * 32 + n;
#pragma unroll
        for (int u = 0; u < (PV == 0 ? 2 : 4); ++u) {
            const int ch = (PV == 0 ? 2 : 4) * hh + u;
            vf.f[cb][u] = *reinterpret_cast<const v4i*>(vs + row * C::VROW + swz<C::VROW>(row, ch) * 16);
        }
    }
}

// P of one tile for one row block, as the P.V B operand.  FP8: w holds the
// lane's 32 codes (byte 4*v + e = accumulator block v/4, register
// 4*(v%4) + e).  fp16/bf16: h[u] holds the 8 values of accumulator block u/2,
// registers 8*(u%2) .. +7.
template <int PV> struct PHalf;
template <> struct PHalf<0> { v8i w; };
template <> struct PHalf<1> { v8h h[4]; };
template <> struct PHalf<2> { v8bf h[4]; };

template <int PV>
__device__ __forceinline__ void phalf_zero(PHalf<PV>& P) {
    if constexpr (PV == 0) {
#pragma unroll
        for (int w = 0; w < 8; ++w) P.w[w] = 0;
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) P.h[u][e] = 0;
    }
}

// Keeps the computation of P inside the block that issues the MFMAs it must
// overlap with (the compiler would otherwise sink it towards its use in the
// next tile, past the rescale branch).
template <int PV>
__device__ __forceinline__ void keep_here(const PHalf<PV>& P) {
#if __HIP_DEVICE_COMPILE__                              // VGPR constraints exist only for the gfx950 pass
    if constexpr (PV == 0) {
        asm volatile("" ::"v"(P.w));
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) asm volatile("" ::"v"(P.h[u]));
    }
#endif
}

// The MFMA "ones" operand of the row-sum product (see rowsum_parity).
template <int PV> struct Ones;
template <> struct Ones<0> { v8i v; };
template <> struct Ones<1> { v8h v; };
template <> struct Ones<2> { v8bf v; };

template <int PV>
__device__ __forceinline__ void make_ones(Ones<PV>& o, bool par) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if constexpr (PV == 0) o.v[e] = par ? 0x38383838 : 0;   // E4M3 1.0 = 0x38
        else if constexpr (PV == 1) o.v[e] = par ? (_Float16)1.0f : (_Float16)0.0f;
        else o.v[e] = par ? (__bf16)1.0f : (__bf16)0.0f;
    }
}

// O^T += V^T P^T and l += rowsum(P) for one row block.
template <int DP, int PV>
__device__ __forceinline__ void pv_half(const VFrag<DP, PV>& vf, const PHalf<PV>& P, const Ones<PV>& ones,
                                        v16f (&o)[DP / 32], v4f& ls) {
    if constexpr (PV == 0) {
#pragma unroll
        for (int cb = 0; cb < DP / 32; ++cb) {
            const v4i lo = vf.f[cb][0], hi = vf.f[cb][1];
            const v8i va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, P.w, o[cb], 0, 0, 0, 0, 0, 0);
        }
        ls = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones.v, P.w, ls, 0, 0, 0, 0, 0, 0);
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int cb = 0; cb < DP / 32; ++cb) {
                if constexpr (PV == 1)
                    o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, vf.f[cb][u]), P.h[u],
                                                                   o[cb], 0, 0, 0);
                else
                    o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, vf.f[cb][u]), P.h[u],
                                                                    o[cb], 0, 0, 0);
            }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if constexpr (PV == 1) ls = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones.v, P.h[u], ls, 0, 0, 0);
            else ls = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones.v, P.h[u], ls, 0, 0, 0);
        }
    }
}

// Online softmax of one tile for one row block (rows row0 + n).
//   f = (q_scale * sm_scale * log2 e) * k_scale per key-scale group g
//   (g = 2*kb + i/8 covers keys 16g .. 16g+15; a 64-key group fills all four),
//   tile max  mt = max over keys of fl32(S * f),
//   raise     iff mt > fl32(m + kTau)  (then m = mt),
//   P         = 2^x,  x = fl32((B + S) * f + fl32(nb - B * f)),
//             nb = log2(P scale) - m,
// exactly as the oracle orders these roundings.  MASKED hides the keys a
// row may not see (past the sequence end, or after the row when causal).
// Returns, per lane, whether its row raised its maximum; m_prev then holds
// the maximum before this tile.
template <int PV, bool MASKED>
__device__ __forceinline__ bool softmax_half(const v16i (&S)[2], const float (&ksv)[4], float cq, float& m_ref,
                                             float& m_prev, PHalf<PV>& P, int k0, int Lk, bool causal, int row,
                                             int hh) {
    constexpr float p_log2_scale = PV == 0 ? kLog2_448 - (float)kTau : 0.f;
    bool vis[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if constexpr (MASKED) {
                const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
                vis[kb][i] = key < Lk && (!causal || key <= row);
            } else {
                vis[kb][i] = true;
            }
        }
    float f[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) f[g] = ksv[g] * cq;
    float smax = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int kb = g >> 1, i0 = (g & 1) * 8;
        int mi = vis[kb][i0] ? S[kb][i0] : kNegInfBits;
#pragma unroll
        for (int i = 1; i < 8; ++i) mi = max(mi, vis[kb][i0 + i] ? S[kb][i0 + i] : kNegInfBits);
        float sg = (bits_f(mi) - kAccBias) * f[g];
        if constexpr (MASKED) sg = mi == kNegInfBits ? -INFINITY : sg;
        smax = fmaxf(smax, sg);
    }
    smax = swap_half_max(smax);
    m_prev = m_ref;
    const bool raise = smax > m_ref + (float)kTau;
    m_ref = raise ? smax : m_ref;
    // a row that has seen no key keeps m = -inf; its P is 0 below
    const float m_use = MASKED ? (m_ref == -INFINITY ? 0.f : m_ref) : m_ref;
    const float nb = p_log2_scale - m_use;
    float cg[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) cg[g] = __builtin_fmaf(-kAccBias, f[g], nb);
    float p[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int g = 2 * kb + (i >> 3);
            float x = __builtin_fmaf(bits_f(S[kb][i]), f[g], cg[g]);
            if constexpr (MASKED) x = vis[kb][i] ? x : -INFINITY;
            p[kb][i] = __builtin_amdgcn_exp2f(x);
        }
    if constexpr (PV == 0) {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int kb = w >> 2, i0 = (w & 3) * 4;
            // the first conversion fills bytes 0-1, the second bytes 2-3
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][i0], p[kb][i0 + 1], __float_as_int(p[kb][i0]), false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][i0 + 2], p[kb][i0 + 3], word, true);
            P.w[w] = word;
        }
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kb = u >> 1, i0 = (u & 1) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (PV == 1) P.h[u][e] = (_Float16)p[kb][i0 + e];
                else P.h[u][e] = (__bf16)p[kb][i0 + e];
            }
        }
    }
    return raise;
}

// Rescale O and l of a row whose maximum moved (m_prev -> m_ref).
template <int DP>
__device__ __forceinline__ void rescale_half(float m_ref, float m_prev, v16f (&o)[DP / 32], v4f& ls) {
    // 0 when the row had no maximum yet (its O and l are 0)
    const float alpha = m_prev == m_ref ? 1.f : __builtin_amdgcn_exp2f(m_prev - m_ref);
#pragma unroll
    for (int cb = 0; cb < DP / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) ls[i] *= alpha;
}

// Instruction order of one pipelined tile (two phases).  Each phase: its K
// fragment reads, then its MFMAs spread evenly through the softmax VALU
// stream of the other row block.  The V fragments are read at the start.
template <int DP, int PV>
__device__ __forceinline__ void interleave_hint() {
    constexpr int NCB = DP / 32;
    constexpr int N_K = 2 * NCB;                                // K fragment reads per phase
    constexpr int N_V = NCB * (PV == 0 ? 2 : 4);                // V fragment reads per tile
    constexpr int N_MFMA = 2 * NCB + (PV == 0 ? NCB + 1 : 4 * NCB + 4);   // per phase
    constexpr int N_VALU = 160;                                 // per phase, approximate
    constexpr int PER = (N_VALU + N_MFMA - 1) / N_MFMA;
    __builtin_amdgcn_sched_group_barrier(0x100, N_K + N_V + 1, 0);   // DS reads: K scales, V, K of phase A
    __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
#pragma unroll
    for (int i = 0; i < N_MFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, PER, 0); // VALU
    }
    __builtin_amdgcn_sched_group_barrier(0x100, N_K, 0);     // DS reads: K of phase B
#pragma unroll
    for (int i = 0; i < N_MFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
    }
}

template <int DP, int PV, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(AttnArgs a) {
    using C = AttnCfg<DP, PV>;
    constexpr int NCB = C::NCB;
    // LDS ring: during step t the wavefronts read K of tile t+1 and V of tile
    // t-1 while tiles t+2 .. t+AHEAD are in flight, so NST = AHEAD + 2.
    constexpr int AHEAD = 3;
    constexpr int NST = AHEAD + 2;
    constexpr int LPT = C::NI + 1;                      // DMA instructions per wavefront per tile
    __shared__ __attribute__((aligned(16))) uint8_t smem[NST * C::STAGE];

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
    // tiles in which no row of the workgroup hides a key: the pipelined loop
    const int n_main = (a.causal ? min(q0, Lk) : Lk) / kBK;

    // ---- per-lane query state: rows wq0 + 32j + n, j = 0, 1
    const int wq0 = q0 + wave * 64;
    const bool live = wq0 < Lq;                         // the wavefront has rows to compute (then wq0 + 63 < nq_pad)
    const int64_t qhead = (int64_t)b * a.Hq + h;
    v4i qf[2][NCB];
    float cq[2], qscale[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int qrow = wq0 + 32 * j + n;
        if (live) {
            const int8_t* q8row = a.q8 + (qhead * a.nq_pad + qrow) * DP;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) qf[j][cb] = *reinterpret_cast<const v4i*>(q8row + cb * 32 + hh * 16);
            qscale[j] = a.qs[qhead * (a.nq_pad >> a.gq_shift) + (qrow >> a.gq_shift)];
        } else {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) qf[j][cb] = v4i{0, 0, 0, 0};
            qscale[j] = 0.f;
        }
        cq[j] = (qscale[j] * a.sm_scale) * kLog2e;      // log2-domain factor of this row
    }

    const int64_t khead = (int64_t)b * a.Hkv + hk;
    const int8_t* kbase = a.k8 + khead * a.nk_pad * DP;
    const float* ksbase = a.ks + khead * (a.nk_pad >> a.gk_shift);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vt) + khead * DP * a.nk_pad * C::VE;
    const int64_t vrow_stride = (int64_t)a.nk_pad * C::VE;
    const bool ks16 = a.gk_shift == 4;                  // K scale groups of 16 keys (else 64)

    v16f o[2][NCB];
    v4f ls[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[j][cb][i] = 0.f;
        ls[j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    float m_ref[2] = {-INFINITY, -INFINITY}, m_prev[2];
    v16i biasv;
#pragma unroll
    for (int i = 0; i < 16; ++i) biasv[i] = kAccBiasBits;
    Ones<PV> ones;
    make_ones<PV>(ones, rowsum_parity(lane));

    auto stage_of = [&](int t) { return smem + (t % NST) * C::STAGE; };
    auto ks_of = [&](const uint8_t* st, float (&ksv)[4]) {
        const v4f k4 = *reinterpret_cast<const v4f*>(st + C::SC_OFF + wave * 16);
#pragma unroll
        for (int g = 0; g < 4; ++g) ksv[g] = k4[g];
    };
    auto issue = [&](int t) {
        if (t < ntiles)
            dma_tile<DP, PV>(stage_of(t), kbase, vbase, vrow_stride, ksbase, ks16, t, wave, lane);
    };
    // end of step t: tile t+2 (read in step t+1) has landed in every wavefront
    auto step_end = [&](int t) {
        if (t + AHEAD < ntiles) wait_vmcnt<LPT * (AHEAD - 2)>();
        else wait_vmcnt<0>();
        block_sync();
    };

    // ---- prologue: tiles 0 .. AHEAD-1 in flight; wait for tiles 0 and 1
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) issue(u);
    if (ntiles >= AHEAD) wait_vmcnt<LPT * (AHEAD - 2)>();
    else wait_vmcnt<0>();
    block_sync();

    // ---- pipelined main loop over the unmasked tiles.  The two row blocks
    // of the wavefront alternate, so that the VALU and the matrix cores always
    // have independent work.  Tile t is one straight-line block:
    //   phase A: softmax of block 0 (tile t)
    //            || QK^T of block 1 (tile t), P.V of block 0 (tile t-1)
    //   phase B: softmax of block 1 (tile t)
    //            || QK^T of block 0 (tile t+1), P.V of block 1 (tile t-1)
    // then, rarely, the rescale of O and l for rows whose maximum moved.  All
    // P.V products issued in tile t use P of tile t-1, computed with the
    // maxima before tile t, so the rescale after them is exact bookkeeping.
    v16i S[2][2];
    PHalf<PV> P[2];
    phalf_zero<PV>(P[0]);                               // P.V of "tile -1" adds exact zeros
    phalf_zero<PV>(P[1]);
    if (n_main > 0 && live) {
        v4i kf[2][NCB];
        load_kfrag<DP>(stage_of(0), n, hh, kf);
        qk_half<DP>(kf, qf[0], biasv, S[0]);
    }
    for (int t = 0; t < n_main; ++t) {
        issue(t + AHEAD);
        if (live) {
            const uint8_t* st = stage_of(t);
            float ksv[4];
            ks_of(st, ksv);
            VFrag<DP, PV> vf;                           // V of tile t-1 (tile 0 for t = 0: times zero P)
            load_vfrag<DP, PV>(stage_of(t == 0 ? 0 : t - 1) + C::KT_BYTES, n, hh, vf);
            const PHalf<PV> P0 = P[0], P1 = P[1];
            bool raised;
            {   // phase A
                v4i kf[2][NCB];
                load_kfrag<DP>(st, n, hh, kf);
                raised = softmax_half<PV, false>(S[0], ksv, cq[0], m_ref[0], m_prev[0], P[0], 0, 0, false, 0, hh);
                qk_half<DP>(kf, qf[1], biasv, S[1]);
                pv_half<DP, PV>(vf, P0, ones, o[0], ls[0]);
            }
            {   // phase B
                v4i kf[2][NCB];
                load_kfrag<DP>(stage_of(t + 1), n, hh, kf);
                raised |= softmax_half<PV, false>(S[1], ksv, cq[1], m_ref[1], m_prev[1], P[1], 0, 0, false, 0, hh);
                qk_half<DP>(kf, qf[0], biasv, S[0]);
                pv_half<DP, PV>(vf, P1, ones, o[1], ls[1]);
            }
            interleave_hint<DP, PV>();
            keep_here<PV>(P[0]);
            keep_here<PV>(P[1]);
            if (__any(raised)) {
                rescale_half<DP>(m_ref[0], m_prev[0], o[0], ls[0]);
                rescale_half<DP>(m_ref[1], m_prev[1], o[1], ls[1]);
            }
        }
        step_end(t);
    }
    if (live && n_main > 0) {                           // P.V of the last pipelined tile
        VFrag<DP, PV> vf;
        load_vfrag<DP, PV>(stage_of(n_main - 1) + C::KT_BYTES, n, hh, vf);
        pv_half<DP, PV>(vf, P[0], ones, o[0], ls[0]);
        pv_half<DP, PV>(vf, P[1], ones, o[1], ls[1]);
    }

    // ---- remaining tiles (a ragged end, the causal diagonal): one at a time
    for (int t = n_main; t < ntiles; ++t) {
        issue(t + AHEAD);
        const int k0 = t * kBK;
        if (live && (!a.causal || k0 <= wq0 + 63)) {
            const uint8_t* st = stage_of(t);
            float ksv[4];
            ks_of(st, ksv);
            v4i kf[2][NCB];
            load_kfrag<DP>(st, n, hh, kf);
            qk_half<DP>(kf, qf[0], biasv, S[0]);
            qk_half<DP>(kf, qf[1], biasv, S[1]);
            const bool need_mask = (k0 + kBK > Lk) || (a.causal && k0 + kBK - 1 > wq0);
            bool raised[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (need_mask)
                    raised[j] = softmax_half<PV, true>(S[j], ksv, cq[j], m_ref[j], m_prev[j], P[j], k0, Lk,
                                                       a.causal, wq0 + 32 * j + n, hh);
                else
                    raised[j] = softmax_half<PV, false>(S[j], ksv, cq[j], m_ref[j], m_prev[j], P[j], k0, Lk,
                                                        a.causal, wq0 + 32 * j + n, hh);
            }
            if (__any(raised[0] || raised[1])) {
                rescale_half<DP>(m_ref[0], m_prev[0], o[0], ls[0]);
                rescale_half<DP>(m_ref[1], m_prev[1], o[1], ls[1]);
            }
            VFrag<DP, PV> vf;
            load_vfrag<DP, PV>(st + C::KT_BYTES, n, hh, vf);
            pv_half<DP, PV>(vf, P[0], ones, o[0], ls[0]);
            pv_half<DP, PV>(vf, P[1], ones, o[1], ls[1]);
        }
        step_end(t);
    }
    if (!live) return;

    // ---- epilogue: normalise, add back V's mean, write in the caller's layout
    const float* vsc = PV == 0 ? a.vs + khead * DP : nullptr;
    const float* vmu = a.vmean ? a.vmean + khead * DP : nullptr;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int qrow = wq0 + 32 * j + n;
        const float l_tot = ls[j][0];                   // the row-sum MFMA covers both lane halves
        const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (qrow < Lq) {
            uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) +
                             (a.cu_q ? (int64_t)(qoff + qrow) * a.on + (int64_t)h * a.oh
                                     : (int64_t)b * a.ob + (int64_t)h * a.oh + (int64_t)qrow * a.on);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int c0 = cb * 32 + 8 * r4 + 4 * hh;
                    if (c0 >= a.d) continue;
                    uint16_t hv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = c0 + e;
                        float val = o[j][cb][4 * r4 + e];
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
            constexpr float p_log2_scale = PV == 0 ? kLog2_448 - (float)kTau : 0.f;
            float part = 0.f;
            if (a.kmean) {
                const float* km = a.kmean + khead * DP;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int code = (int)(int8_t)((qf[j][cb][e >> 2] >> (8 * (e & 3))) & 0xff);
                        part += (float)code * km[cb * 32 + hh * 16 + e];
                    }
            }
            const float dot = swap_half_sum(part);
            if (hh == 0 && qrow < Lq) {
                const float corr = a.kmean ? a.sm_scale * qscale[j] * dot : 0.f;
                const float lse = (m_ref[j] + __log2f(l_tot) - p_log2_scale) * kLn2 + corr;
                const int64_t li = a.lse_varlen ? (int64_t)h * a.total_q + qoff + qrow : qhead * a.Nq + qrow;
                a.lse[li] = lse;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Exact int32 scores from the same K staging and QK^T fragment code, for
// tests.  One workgroup covers kDbgBQ query rows (32 per wavefront).
constexpr int kDbgBQ = 128;

template <int DP>
__global__ __launch_bounds__(kThreads) void qk_scores_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t ks[kBK * DP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int nqt = (a.Nq + kDbgBQ - 1) / kDbgBQ;
    const int qt = blockIdx.x % nqt, bh = blockIdx.x / nqt, h = bh % a.Hq, b = bh / a.Hq;
    const int hk = h / (a.Hq / a.Hkv);
    const int qrow = qt * kDbgBQ + wave * 32 + n;
    const int64_t qhead = (int64_t)b * a.Hq + h;
    const int8_t* q8row = a.q8 + (qhead * a.nq_pad + qrow) * DP;
    // the same fragment code as the attention kernel, with both row blocks
    // holding this wavefront's 32 rows
    v4i qf[2][DP / 32];
#pragma unroll
    for (int cb = 0; cb < DP / 32; ++cb)
        qf[0][cb] = qf[1][cb] = *reinterpret_cast<const v4i*>(q8row + cb * 32 + hh * 16);
    const int8_t* kbase = a.k8 + ((int64_t)b * a.Hkv + hk) * a.nk_pad * DP;
    const int ntiles = (a.Nk + kBK - 1) / kBK;
    unsigned long long s1 = 0, s2 = 0;
    v16i biasv;
#pragma unroll
    for (int i = 0; i < 16; ++i) biasv[i] = kAccBiasBits;
    constexpr int KCPR = DP / 16, K_LOADS = kBK * DP / (16 * kThreads);
    for (int t = 0; t < ntiles; ++t) {
        uint4 kr[K_LOADS];
        const uint4* ksrc = reinterpret_cast<const uint4*>(kbase + (int64_t)t * kBK * DP);
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) kr[i] = ksrc[i * kThreads + tid];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int L = i * kThreads + tid, row = L / KCPR, ch = L % KCPR;
            *reinterpret_cast<uint4*>(ks + row * DP + swz<DP>(row, ch) * 16) = kr[i];
        }
        __syncthreads();
        v4i kf[2][DP / 32];
        load_kfrag<DP>(ks, n, hh, kf);
        v16i acc[2][2];
        qk_half<DP>(kf, qf[0], biasv, acc[0]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = t * kBK + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
                const int S = acc[0][kb][i] - kAccBiasBits;
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

hipError_t launch_attn(const AttnArgs& a_in, int dp, int pv, bool out_bf16, hipStream_t s) {
    AttnArgs a = a_in;
    a.n_qtiles = (a.Nq + kBQ - 1) / kBQ;
    a.num_wg = a.B * a.Hq * a.n_qtiles;
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
    const int grid = a.B * a.Hq * ((a.Nq + kDbgBQ - 1) / kDbgBQ);
    if (dp == 128) qk_scores_kernel<128><<<grid, kThreads, 0, s>>>(a);
    else qk_scores_kernel<64><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sage
