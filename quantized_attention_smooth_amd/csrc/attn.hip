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
//  * the running maximum follows the plain online-softmax update: a row's
//    reference maximum becomes max(m, tile maximum) and O^T (fp32) and the
//    row sums are rescaled by 2^(m - m') whenever some row of the wavefront
//    moved it.
#include <type_traits>

#include "sage_device.h"

namespace sage {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2 of the FP8 P scale (448)
// log2 of P's static scale: 448 puts p = 2^(s - m') <= 1 at the top of the FP8
// range; the fp16/bf16 operand takes p itself
template <int PV>
constexpr float kPLog2Scale = PV == 0 ? kLog2_448 : 0.f;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Compile-time loop: f(std::integral_constant<int, i>) for i = I .. N-1.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}
typedef float v4f __attribute__((ext_vector_type(4)));

// A value the whole wavefront shares, moved to scalar registers.  Head and
// batch indices come out of integer divisions, which the compiler evaluates
// with vector instructions; buffer resources built from such values would
// stay in vector registers and every buffer load would need a loop over the
// lanes' distinct resources.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <class T>
__device__ __forceinline__ T* uniform(T* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

template <int DP, int PV, int NW = 4, int NR = NW>
struct AttnCfg {
    static constexpr int NCB = DP / 32;                 // 32-channel blocks
    static constexpr int KT_BYTES = kBK * DP;           // K tile: 64 keys x Dp int8
    static constexpr int VE = PV == 0 ? 1 : 2;          // V element bytes
    static constexpr int VROW = kBK * VE;               // V^T tile row (one channel) bytes
    static constexpr int VT_BYTES = DP * VROW;
    static constexpr int SC_BYTES = NR * 256;           // the tile's K scales, one 256-byte slot per reading wavefront
    static constexpr int STAGE = KT_BYTES + VT_BYTES + SC_BYTES;
    static constexpr int NI = (KT_BYTES + VT_BYTES) / (16 * 64 * NW);   // tile DMA instructions per copying wavefront
    static constexpr int NSC = NR / NW;                 // scale copies per copying wavefront
    static_assert(NI * 16 * 64 * NW == KT_BYTES + VT_BYTES, "tile must fill whole copy rounds");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// One stage of the LDS ring of NST stages.  The ring keeps its K tiles, its
// V^T tiles and its K-scale slots in three regions (all K tiles first, then
// all V^T tiles, then all scale slots), so that within each region every
// stage is a constant offset below 64 KB from one base address.
struct StagePtrs {
    uint8_t* k;                                         // K tile
    uint8_t* v;                                         // V^T tile
    uint8_t* s;                                         // K-scale slots
};
template <class C, int NST>
__device__ __forceinline__ StagePtrs ring_stage(uint8_t* smem, int u) {
    return {smem + u * C::KT_BYTES, smem + NST * C::KT_BYTES + u * C::VT_BYTES,
            smem + NST * (C::KT_BYTES + C::VT_BYTES) + u * C::SC_BYTES};
}
// The 4-wave kernel's ring keeps each stage's K tile, V^T tile and scale
// slots together, in that order.
template <class C>
__device__ __forceinline__ StagePtrs ring_stage_packed(uint8_t* smem, int u) {
    uint8_t* st = smem + u * C::STAGE;
    return {st, st + C::KT_BYTES, st + C::KT_BYTES + C::VT_BYTES};
}

// Direct global -> LDS copy of one key tile into one stage of the ring, as
// NI + NSC instructions per copying wavefront that the key loop can place one
// by one.  Instruction i < NI of copying wavefront w (of NW) fills the 1 KB of
// granules [(NW*i + w) * 64, +64) of the tile (K granules first, then V^T
// granules, each in its own region of the stage); lane L writes granule
// (NW*i + w) * 64 + L.
// The granule at (row, physical chunk c) receives logical chunk swz(row, c)
// (the swizzle is an involution), so readers address logical chunk c at
// swz(row, c).  Instruction NI + j copies the tile's K scales into the 256-byte
// slot of reading wavefront w + NW*j, 4 bytes per lane: lane L holds group
// L % 4 (4 groups of 16 keys), or the one group of 64 keys; the softmax reads
// the first 16 bytes.  All lanes take part so that no branch splits the loop
// body.  Whether a wavefront's granules belong to K or to V^T depends only on
// the instruction and the wavefront, so the choice is wave-uniform.
template <int DP, int PV, int NW = 4, int NR = NW>
struct TileCopy {
    const int8_t* kbase;
    const uint8_t* vbase;
    int64_t vrow_stride;
    const float* ksbase;
    bool ks16;
    int wave, lane;                                     // wave is wave-uniform (an SGPR)

    template <int I>
    __device__ __forceinline__ void issue(const StagePtrs& stage, int t) const {
        using C = AttnCfg<DP, PV, NW, NR>;
        constexpr int KG = C::KT_BYTES / 16, KCPR = DP / 16, VCPR = C::VROW / 16;
        static_assert(KG % 64 == 0, "K tile must fill whole wavefront chunks");
        if constexpr (I < C::NI) {
            const int gbase = (NW * I + wave) * 64;
            const int g = gbase + lane;
            auto k_src = [&]() {
                const int row = g / KCPR, ch = swz<DP>(row, g % KCPR);
                return reinterpret_cast<const uint8_t*>(kbase) + (int64_t)t * C::KT_BYTES + row * DP + ch * 16;
            };
            auto v_src = [&]() {
                const int gv = g - KG, row = gv / VCPR, ch = swz<C::VROW>(row, gv % VCPR);
                return vbase + row * vrow_stride + (int64_t)t * C::VROW + ch * 16;
            };
            const uint8_t* src;
            uint8_t* dst;
            if constexpr ((I + 1) * NW * 64 <= KG) src = k_src(), dst = stage.k + gbase * 16;
            else if constexpr (I * NW * 64 >= KG) src = v_src(), dst = stage.v + (gbase - KG) * 16;
            else if (gbase < KG) src = k_src(), dst = stage.k + gbase * 16;
            else src = v_src(), dst = stage.v + (gbase - KG) * 16;
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)dst, 16, 0, 0);
        } else {
            const float* src = ks16 ? ksbase + 4 * t + (lane & 3) : ksbase + t;
            const int slot = wave + NW * (I - C::NI);
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(stage.s + slot * 256), 4, 0, 0);
        }
    }
    __device__ __forceinline__ void issue_all(const StagePtrs& stage, int t) const {
        using C = AttnCfg<DP, PV, NW, NR>;
        static_for<0, C::NI + C::NSC>([&](auto i) { issue<decltype(i)::value>(stage, t); });
    }
};

// The same copy through buffer resources: every source address is a 32-bit
// per-lane offset (one VGPR per instruction, fixed for the whole key loop)
// plus a wave-uniform offset for the tile, and the hardware clamps each load
// to its resource (bytes past the end read as zero).
#if __HIP_DEVICE_COMPILE__
template <int DP, int PV, int NW, int NR>
struct TileCopyBuf {
    using C = AttnCfg<DP, PV, NW, NR>;
    __amdgpu_buffer_rsrc_t rk, rv, rs;
    uint32_t voff[C::NI + 1];
    int wave;
    bool ks16;

    __device__ __forceinline__ TileCopyBuf(const int8_t* kbase, const uint8_t* vbase, uint32_t vrow_stride,
                                           const float* ksbase, uint32_t k_bytes, uint32_t v_bytes,
                                           uint32_t s_bytes, bool ks16_, int wave_, int lane)
        : wave(wave_), ks16(ks16_) {
        constexpr int KG = C::KT_BYTES / 16, KCPR = DP / 16, VCPR = C::VROW / 16;
        rk = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, (int)k_bytes, 0x00020000);
        rv = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, (int)v_bytes, 0x00020000);
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)ksbase, (short)0, (int)s_bytes, 0x00020000);
#pragma unroll
        for (int i = 0; i < C::NI; ++i) {
            const int g = (NW * i + wave) * 64 + lane;
            if (g < KG) {
                const int row = g / KCPR, ch = swz<DP>(row, g % KCPR);
                voff[i] = (uint32_t)(row * DP + ch * 16);
            } else {
                const int gv = g - KG, row = gv / VCPR, ch = swz<C::VROW>(row, gv % VCPR);
                voff[i] = (uint32_t)row * vrow_stride + (uint32_t)(ch * 16);
            }
        }
        voff[C::NI] = ks16 ? (uint32_t)(lane & 3) * 4u : 0u;
    }

    template <int I>
    __device__ __forceinline__ void issue(const StagePtrs& stage, int t) const {
        constexpr int KG = C::KT_BYTES / 16;
        if constexpr (I < C::NI) {
            const int gbase = (NW * I + wave) * 64;
            lds_ptr_t kdst = (lds_ptr_t)(stage.k + gbase * 16);
            lds_ptr_t vdst = (lds_ptr_t)(stage.v + (gbase - KG) * 16);
            if constexpr ((I + 1) * NW * 64 <= KG) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, kdst, 16, voff[I], (uint32_t)t * C::KT_BYTES, 0, 0);
            } else if constexpr (I * NW * 64 >= KG) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, vdst, 16, voff[I], (uint32_t)t * C::VROW, 0, 0);
            } else {
                if (gbase < KG) __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, kdst, 16, voff[I], (uint32_t)t * C::KT_BYTES, 0, 0);
                else __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, vdst, 16, voff[I], (uint32_t)t * C::VROW, 0, 0);
            }
        } else {
            const int slot = wave + NW * (I - C::NI);
            lds_ptr_t dst = (lds_ptr_t)(stage.s + slot * 256);
            const uint32_t so = ks16 ? (uint32_t)t * 16u : (uint32_t)t * 4u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voff[C::NI], so, 0, 0);
        }
    }
    __device__ __forceinline__ void issue_all(const StagePtrs& stage, int t) const {
        static_for<0, C::NI + C::NSC>([&](auto i) { issue<decltype(i)::value>(stage, t); });
    }
};
#else
// Host pass: the buffer builtins exist only for the gfx950 target; this
// interface-only stand-in lets the kernel body parse.
template <int DP, int PV, int NW, int NR>
struct TileCopyBuf {
    __device__ TileCopyBuf(const int8_t*, const uint8_t*, uint32_t, const float*, uint32_t, uint32_t, uint32_t, bool,
                           int, int) {}
    template <int I> __device__ void issue(const StagePtrs&, int) const {}
    __device__ void issue_all(const StagePtrs&, int) const {}
};
#endif

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Waits until this wavefront's LDS accesses are done.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier that also keeps the compiler from moving LDS accesses
// across it (the hardware ordering comes from the explicit vmcnt waits).
__device__ __forceinline__ void block_sync() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Stores channels c0 .. c0+3 (those below d) of one output row at element
// offset `row_off` of out: fp32 values (split-KV partial results) or values
// rounded to fp16/bf16, as one 8-byte (16-byte for fp32) write when vec4.
template <bool OUT_BF16>
__device__ __forceinline__ void store_out4(void* out, bool out_f32, bool vec4, int64_t row_off, int c0, int d,
                                           const float (&val)[4]) {
    if (out_f32) {
        float* o = reinterpret_cast<float*>(out) + row_off + c0;
        if (vec4 && c0 + 3 < d) {
            *reinterpret_cast<float4*>(o) = make_float4(val[0], val[1], val[2], val[3]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c0 + e < d) o[e] = val[e];
        }
        return;
    }
    uint16_t hv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) hv[e] = Half<OUT_BF16>::from_f(val[e]);
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + row_off + c0;
    if (vec4 && c0 + 3 < d) {
        uint2 w;
        w.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
        w.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
        *reinterpret_cast<uint2*>(o) = w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (c0 + e < d) o[e] = hv[e];
    }
}

// Channels c0 .. c0+3 of a per-channel array of one head, padded to Dp
// channels (c0 + 3 < Dp: the reads stay inside the padded row).  Four
// unconditional 4-byte loads (the arrays need only 4-byte alignment); an
// epilogue loads all its factors this way before using any, so that the loads
// are in flight together instead of one round trip each.
__device__ __forceinline__ v4f load_ch4(const float* p, int c0) {
    return v4f{p[c0], p[c0 + 1], p[c0 + 2], p[c0 + 3]};
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

// First MFMA of a score chain: K.Q^T of one channel block plus the
// accumulator bias, which enters as the inline constant 1/(2 pi) (the bits
// kAccBiasBits) and so needs no registers.  It is inline assembly because
// the compiler hoists a constant accumulator operand out of the key loop into
// registers instead of encoding it.  The destination is early-clobber: an
// MFMA may not write registers it is still reading.  The compiler's hazard
// checks do not look inside inline assembly, so the statement brings its own
// two wait states for a VALU instruction that writes a or b just before it
// (the compiler places such copies, e.g. from AGPRs).  Its result is read
// only by the next MFMA of the same chain, as the accumulator of the same
// opcode, which the hardware forwards.
static_assert(kAccBiasBits == 0x3E22F983, "the inline constant below is these bits");
__device__ __forceinline__ v16i mfma_i8_biased(const v4i& a, const v4i& b) {
    v16i d;
    asm("s_nop 1\n\tv_mfma_i32_32x32x32_i8 %0, %1, %2, 0.15915494" : "=&v"(d) : "v"(a), "v"(b));
    return d;
}

// S^T of one row block: S[kb][i] = bias + S(query n of the block,
// key 32*kb + 8*(i/4) + 4*hh + i%4).  Two accumulation chains over the
// channel blocks; the first MFMA of each adds the accumulator bias.
template <int DP>
__device__ __forceinline__ void qk_half(const v4i (&kf)[2][DP / 32], const v4i (&qf)[DP / 32], v16i (&S)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) S[kb] = mfma_i8_biased(kf[kb][0], qf[0]);
#pragma unroll
    for (int cb = 1; cb < DP / 32; ++cb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            S[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kb][cb], qf[cb], S[kb], 0, 0, 0);
}

// V^T operand of P.V for one tile.  FP8: a[cb] = the 32 bytes of channel row cb*32 + n for the keys of
// lane half hh; fp16/bf16: a[cb][u] = 8 of those keys (u-th 16-byte chunk).
template <int DP, int PV> struct VA;
template <int DP> struct VA<DP, 0> { v8i a[DP / 32]; };
template <int DP> struct VA<DP, 1> { v4i a[DP / 32][4]; };
template <int DP> struct VA<DP, 2> { v4i a[DP / 32][4]; };

template <int DP, int PV>
__device__ __forceinline__ void load_va(const uint8_t* vs, int n, int hh, VA<DP, PV>& va) {
    using C = AttnCfg<DP, PV>;
#pragma unroll
    for (int cb = 0; cb < DP / 32; ++cb) {
        const int row = cb * 32 + n;
        const uint8_t* r = vs + row * C::VROW;
        if constexpr (PV == 0) {
            const v4i lo = *reinterpret_cast<const v4i*>(r + swz<C::VROW>(row, 2 * hh) * 16);
            const v4i hi = *reinterpret_cast<const v4i*>(r + swz<C::VROW>(row, 2 * hh + 1) * 16);
            va.a[cb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) va.a[cb][u] = *reinterpret_cast<const v4i*>(r + swz<C::VROW>(row, 4 * hh + u) * 16);
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
#if __HIP_DEVICE_COMPILE__                              // register constraints exist only for the gfx950 pass
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

// ---- P.V on the matrix cores with O^T in AGPRs.
// The library is built with MFMA results in VGPRs, so that the softmax reads
// the score accumulators directly; the output accumulators, which only the
// matrix cores touch, live in AGPRs instead, through these MFMAs written as
// inline assembly.  The compiler does not see them as MFMAs, so every place
// where compiled code reads or writes O passes o_guard() first and after:
// an MFMA result may be read by the VALU only 18 wait states after a 16-pass
// MFMA, and a VALU write must precede the MFMA that reads it by a few.
template <int DP>
__device__ __forceinline__ void o_guard(v16f (&o)[DP / 32]) {
#if __HIP_DEVICE_COMPILE__
    if constexpr (DP == 128)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0]), "+a"(o[1]));
#endif
}

// Keeps the P.V operands (V^T and P) alive and untouched
// until a safe distance after the last MFMA that reads them: an MFMA may
// still be waiting behind the previous one on the matrix core when the
// compiler, which sees only inline assembly, would reuse those registers.
template <int DP, int PV>
__device__ __forceinline__ void operands_guard(VA<DP, PV>& va, PHalf<PV>& p0, PHalf<PV>& p1) {
#if __HIP_DEVICE_COMPILE__
    if constexpr (PV == 0) {
#pragma unroll
        for (int cb = 0; cb < DP / 32; ++cb) asm volatile("" : "+v"(va.a[cb]));
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(p0.w), "+v"(p1.w));
#pragma unroll
        for (int cb = 0; cb < DP / 32; ++cb) asm volatile("" : "+v"(va.a[cb]));
    } else {
#pragma unroll
        for (int cb = 0; cb < DP / 32; ++cb)
#pragma unroll
            for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(va.a[cb][u]));
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(p0.h[0]), "+v"(p0.h[1]), "+v"(p0.h[2]), "+v"(p0.h[3]),
                     "+v"(p1.h[0]), "+v"(p1.h[1]), "+v"(p1.h[2]), "+v"(p1.h[3]));
#pragma unroll
        for (int cb = 0; cb < DP / 32; ++cb)
#pragma unroll
            for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(va.a[cb][u]));
    }
#endif
}

// One P.V MFMA: O^T[cb] += V^T[cb] P^T (FP8: all 64 keys; fp16/bf16: the
// 16-key slice u).  The V^T operand comes from LDS loads whose lgkmcnt wait
// the compiler places right before this instruction, or from VALU writes it
// cannot see as hazards here; the matrix core needs a few more wait states
// before it reads such registers (without them the first MFMA after the wait
// was seen to read stale values), hence the s_nop inside the statement.
template <int DP, int PV, int CB, int U>
__device__ __forceinline__ void pv_job(const VA<DP, PV>& va, const PHalf<PV>& P, v16f (&o)[DP / 32]) {
#if __HIP_DEVICE_COMPILE__
    if constexpr (PV == 0)
        asm("s_nop 4\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(o[CB]) : "v"(va.a[CB]), "v"(P.w));
    else if constexpr (PV == 1)
        asm("s_nop 4\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(o[CB]) : "v"(va.a[CB][U]), "v"(P.h[U]));
    else
        asm("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o[CB]) : "v"(va.a[CB][U]), "v"(P.h[U]));
#endif
}

// Row sums: l += rowsum(P) (slice U on the fp16/bf16 path).
template <int PV, int U>
__device__ __forceinline__ void rs_job(const PHalf<PV>& P, const Ones<PV>& ones, v4f& ls) {
    if constexpr (PV == 0) ls = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones.v, P.w, ls, 0, 0, 0, 0, 0, 0);
    else if constexpr (PV == 1) ls = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones.v, P.h[U], ls, 0, 0, 0);
    else ls = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones.v, P.h[U], ls, 0, 0, 0);
}

// The whole P.V and row-sum step of one row block (outside the pipeline).
template <int DP, int PV>
__device__ __forceinline__ void pv_all(const VA<DP, PV>& va, const PHalf<PV>& P, const Ones<PV>& ones,
                                       v16f (&o)[DP / 32], v4f& ls) {
    static_for<0, DP / 32>([&](auto cb) {
        if constexpr (PV == 0) pv_job<DP, PV, decltype(cb)::value, 0>(va, P, o);
        else static_for<0, 4>([&](auto u) { pv_job<DP, PV, decltype(cb)::value, decltype(u)::value>(va, P, o); });
    });
    if constexpr (PV == 0) rs_job<PV, 0>(P, ones, ls);
    else static_for<0, 4>([&](auto u) { rs_job<PV, decltype(u)::value>(P, ones, ls); });
}

// Online softmax of one tile for one row block (rows row + n).
//   f = (q_scale * sm_scale * log2 e) * k_scale per key-scale group g
//   (g = 2*kb + i/8 covers keys 16g .. 16g+15; a 64-key group fills all four),
//   tile max  mt = max over keys of fl32(S * f),
//   raise     iff mt > m  (then m = mt: m' = max(m, mt)),
//   P         = 2^x,  x = fl32((B + S) * f + fl32(nb - B * f)),
//             nb = log2(P scale) - m, with B + S the score accumulator
//             read as a float (its bias B < 2^24, so B + S is exact).
// MASKED hides the keys a
// row may not see (past the sequence end, or after the row when causal).
// Returns, per lane, whether its row raised its maximum; m_prev then holds
// the maximum before this tile.  (Used by the masked tiles; the pipelined
// loop runs the same steps in pieces, see SoftmaxPieces.)
template <int PV, bool MASKED>
__device__ __forceinline__ bool softmax_half(const v16i (&S)[2], const float (&ksv)[4], float cq, float& m_ref,
                                             float& m_prev, PHalf<PV>& P, int k0, int Lk, bool causal, int row,
                                             int hh) {
    constexpr float p_log2_scale = kPLog2Scale<PV>;
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
    const bool raise = smax > m_ref;
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

// Causal mask of one 32-key half of a tile in the pipelined loop.  Element i
// of the lane's scores is key 8*(i/4) + 4*hh + i%4 of the half; lim is the
// lane's row minus the half's first key minus 4*hh, so the key is visible iff
// its offset 8*(i/4) + i%4 <= lim.  Masked scores become the -inf pattern,
// which no group maximum takes and whose exponent is -inf (P = 0).
__device__ __forceinline__ void causal_mask_half(v16i& Sk, int lim) {
#pragma unroll
    for (int i = 0; i < 16; ++i) Sk[i] = 8 * (i >> 2) + (i & 3) <= lim ? Sk[i] : kNegInfBits;
}

// The unmasked softmax of one row block cut into pieces that the pipelined
// loop interleaves with MFMAs: head<0..3>() compute the scale factors and the
// tile maximum and take the raise decision (the same steps and roundings as
// softmax_half), piece<E>() turns the lane's 32 keys into P two at a time.
// KS16: the tile has four K-scale groups of 16 keys; otherwise one group of
// 64 keys, whose scale the four slots of ksv repeat, so that one scale
// factor, one exponent offset and one maximum serve the whole tile (the same
// values as the four-group steps give: the factor is >= 0, so scaling the
// integer maximum equals the maximum of the scaled groups).
template <int PV, bool KS16 = true>
struct SoftmaxPieces {
    static constexpr float p_log2_scale = kPLog2Scale<PV>;
    float f[4], cg[4], smax;
    int mi[4];
    int word[8];                                        // FP8: bytes 0-1 of word w between its two chunks
    bool raise;

    template <int H>
    __device__ __forceinline__ void head(const v16i (&S)[2], const float (&ksv)[4], float cq, float& m_ref,
                                         float& m_prev) {
        head<H>(S[0], S[1], ksv, cq, m_ref, m_prev);
    }
    template <int H>
    __device__ __forceinline__ void head(const v16i& S0, const v16i& S1, const float (&ksv)[4], float cq,
                                         float& m_ref, float& m_prev) {
        if constexpr (H == 0) {
#pragma unroll
            for (int g = 0; g < 4; ++g) f[g] = ksv[g] * cq;
            group_max(S0, 0);
        } else if constexpr (H == 1) {
            group_max(S0, 1);
            group_max(S1, 2);
        } else if constexpr (H == 2) {
            group_max(S1, 3);
            smax = -INFINITY;
#pragma unroll
            for (int g = 0; g < 4; ++g) smax = fmaxf(smax, (bits_f(mi[g]) - kAccBias) * f[g]);
        } else {
            smax = swap_half_max(smax);
            m_prev = m_ref;
            raise = smax > m_ref;
            m_ref = raise ? smax : m_ref;
            const float nb = p_log2_scale - m_ref;
#pragma unroll
            for (int g = 0; g < 4; ++g) cg[g] = __builtin_fmaf(-kAccBias, f[g], nb);
        }
    }
    // The same head split into calls that the 8-wavefront loop places
    // itself: prep() and gmax() need only the scores, decide() takes the
    // raise decision and the new maximum, spec() gives the exponent offsets
    // for a maximum (same roundings as head<>()).
    __device__ __forceinline__ void prep(const float (&ksv)[4], float cq) {
        if constexpr (KS16) {
#pragma unroll
            for (int g = 0; g < 4; ++g) f[g] = ksv[g] * cq;
        } else {
            const float f0 = ksv[0] * cq;
#pragma unroll
            for (int g = 0; g < 4; ++g) f[g] = f0;
        }
    }
    // A floor of FLT_MIN under the scale factors where scores can be masked:
    // a masked score (the -inf pattern) times a factor of 0 would give NaN,
    // with the floor it gives -inf.  The other exponents keep their values:
    // the floor's products are below half an ulp of the offset they join.
    __device__ __forceinline__ void floor_f() {
#pragma unroll
        for (int g = 0; g < 4; ++g) f[g] = fmaxf(f[g], 1.17549435e-38f);
    }
    __device__ __forceinline__ void gmax(const v16i& Sk, int g) { group_max(Sk, g); }
    __device__ __forceinline__ void spec(float m_ref) {
        const float nb = p_log2_scale - m_ref;
        if constexpr (KS16) {
#pragma unroll
            for (int g = 0; g < 4; ++g) cg[g] = __builtin_fmaf(-kAccBias, f[g], nb);
        } else {
            const float c0 = __builtin_fmaf(-kAccBias, f[0], nb);
#pragma unroll
            for (int g = 0; g < 4; ++g) cg[g] = c0;
        }
    }
    __device__ __forceinline__ void decide(float& m_ref, float& m_prev) {
        if constexpr (KS16) {
            smax = -INFINITY;
#pragma unroll
            for (int g = 0; g < 4; ++g) smax = fmaxf(smax, (bits_f(mi[g]) - kAccBias) * f[g]);
        } else {
            const int m4 = max(max(mi[0], mi[1]), max(mi[2], mi[3]));
            smax = (bits_f(m4) - kAccBias) * f[0];
        }
        smax = swap_half_max(smax);
        m_prev = m_ref;
        raise = smax > m_ref;
        m_ref = raise ? smax : m_ref;
    }

    // Keys 2E and 2E+1 of the lane's 32 become P in three stages, which the
    // loop skews over consecutive pieces (piece e: products of chunk e, exp2
    // of chunk e-1, conversion of chunk e-2), so that no instruction waits
    // for the one just before it.
    static constexpr int NPIECE = 18;
    float xv[32], pv[32];

    template <int E>
    __device__ __forceinline__ void piece(const v16i (&S)[2], PHalf<PV>& P) {
        piece<E>(S[0], S[1], P);
    }
    // Pieces 0-7 read only S0 and pieces 8-15 only S1.
    template <int E>
    __device__ __forceinline__ void piece(const v16i& S0, const v16i& S1, PHalf<PV>& P) {
        if constexpr (E < 16) {
            constexpr int kb = E >> 3, i0 = (2 * E) & 15, g = 2 * kb + (i0 >> 3);
            const v16i& Sk = kb == 0 ? S0 : S1;
            xv[2 * E] = __builtin_fmaf(bits_f(Sk[i0]), f[g], cg[g]);
            xv[2 * E + 1] = __builtin_fmaf(bits_f(Sk[i0 + 1]), f[g], cg[g]);
        }
        if constexpr (E >= 1 && E - 1 < 16) {
            pv[2 * E - 2] = __builtin_amdgcn_exp2f(xv[2 * E - 2]);
            pv[2 * E - 1] = __builtin_amdgcn_exp2f(xv[2 * E - 1]);
        }
        if constexpr (E >= 2) convert<E - 2>(P);
    }

    template <int C>
    __device__ __forceinline__ void convert(PHalf<PV>& P) {
        constexpr int kb = C >> 3, i0 = (2 * C) & 15, g = 2 * kb + (i0 >> 3);
        const float p0 = pv[2 * C], p1 = pv[2 * C + 1];
        if constexpr (PV == 0) {
            constexpr int w = C >> 1;
            if constexpr ((C & 1) == 0) word[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(p0), false);
            else P.w[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, word[w], true);
        } else if constexpr (PV == 1) {
            P.h[g][i0 & 7] = (_Float16)p0;
            P.h[g][(i0 & 7) + 1] = (_Float16)p1;
        } else {
            P.h[g][i0 & 7] = (__bf16)p0;
            P.h[g][(i0 & 7) + 1] = (__bf16)p1;
        }
    }

  private:
    __device__ __forceinline__ void group_max(const v16i& Sk, int g) {
        const int i0 = (g & 1) * 8;
        int m = Sk[i0];
#pragma unroll
        for (int i = 1; i < 8; ++i) m = max(m, Sk[i0 + i]);
        mi[g] = m;
    }
};

// Rescale O and l of a row whose maximum moved (m_prev -> m_ref).  O must be
// guarded (o_guard) around this.
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

// ---- instruction interleave of the pipelined loop
// A region pairs NJ matrix-core jobs (MFMAs) with NV VALU pieces: after job k
// come pieces k*NV/NJ .. (k+1)*NV/NJ - 1, and a scheduling fence keeps the
// compiler from regrouping them, so that one wavefront keeps both the VALU
// and the matrix cores busy.  job(k) and piece(e) take
// std::integral_constant indices.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

template <int NJ, int NV, class J, class V>
__device__ __forceinline__ void interleave(J&& job, V&& piece) {
    static_for<0, NJ>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        job(kc);
        static_for<k * NV / NJ, (k + 1) * NV / NJ>(piece);
        sched_fence();
    });
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

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
    const int n = lane & 31, hh = lane >> 5;

    // ---- work item (the same order as the FP8 kernel: causal calls and
    // varlen batches round-robin over the XCDs, causal longest tiles first)
    const bool lpt = a.causal;
    int wg = (a.cu_q || a.causal) ? (int)blockIdx.x : xcd_remap(blockIdx.x, a.num_wg);
    int split = 0;
    if (a.n_splits > 1) {                               // split-KV: consecutive workgroups, consecutive key ranges
        split = wg % a.n_splits;
        wg /= a.n_splits;
    }
    const int nbh = a.num_wg / (a.n_qtiles * a.n_splits);
    int qt = lpt ? wg / nbh : wg % a.n_qtiles;
    const int bh = lpt ? wg % nbh : wg / a.n_qtiles, h = bh % a.Hq, b = bh / a.Hq;
    if (a.causal) qt = a.n_qtiles - 1 - qt;             // longest rows first
    int Lq = a.Nq, Lk = a.Nk, qoff = 0;
    if (a.cu_q) {                                       // a sequence longer than max_seqlen is cut to it
        qoff = a.cu_q[b];
        Lq = min(max(a.cu_q[b + 1] - qoff, 0), a.Nq);
        Lk = min(max(a.cu_k[b + 1] - a.cu_k[b], 0), a.Nk);
    }
    const int kb0 = split * a.split_len;                // first key of this workgroup's range
    if (a.n_splits > 1) Lk = min(Lk - kb0, a.split_len);
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
        cq[j] = ((qscale[j] * a.sm_scale) * kLog2e) * kAccScale;   // log2-domain factor of this row, times 2^26
    }

    const int64_t khead = (int64_t)b * a.Hkv + hk;
    const int8_t* kbase = a.k8 + khead * a.nk_pad * DP + (int64_t)kb0 * DP;
    const float* ksbase = a.ks + khead * (a.nk_pad >> a.gk_shift) + (kb0 >> a.gk_shift);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vt) + (khead * DP * a.nk_pad + kb0) * C::VE;
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
    Ones<PV> ones;
    make_ones<PV>(ones, rowsum_parity(lane));

    auto stage_of = [&](int t) { return ring_stage_packed<C>(smem, t % NST); };
    auto ks_of = [&](const StagePtrs& st, float (&ksv)[4]) {
        const v4f k4 = *reinterpret_cast<const v4f*>(st.s + wave * 256);
#pragma unroll
        for (int g = 0; g < 4; ++g) ksv[g] = k4[g];
    };
    const TileCopy<DP, PV> copier{kbase, vbase, vrow_stride, ksbase, ks16, wave, lane};
    auto issue = [&](int t) {
        if (t < ntiles) copier.issue_all(stage_of(t), t);
    };
    // end of step t: tile t+2 (read in step t+1) has landed in every wavefront
    auto step_end = [&](int t) {
        if (t + AHEAD < ntiles) wait_vmcnt<LPT * (AHEAD - 2)>();
        else wait_vmcnt<0>();
        block_sync();
    };

    // ---- prologue: tiles 0 .. AHEAD-1 in flight; wait for tiles 0 and 1.
    // The copies are unconditional (past the last tile they copy it again,
    // into stages no step reads), so that the number of loads in flight is
    // the same on every path and the compiler waits for the Q fragments
    // without waiting for the whole prologue.
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) copier.issue_all(stage_of(u), max(min(u, ntiles - 1), 0));
    wait_vmcnt<LPT * (AHEAD - 2)>();
    block_sync();

    // ---- pipelined main loop over the unmasked tiles.  The two row blocks
    // of the wavefront alternate, so that the VALU and the matrix cores always
    // have independent work.  Tile t is four regions (VALU || matrix cores):
    //   H0: maximum of block 0 (tile t)   || P.V of block 1 (tile t-1)
    //   E0: P of block 0 (tile t)         || QK^T of block 1 (tile t)
    //   H1: maximum of block 1 (tile t)   || P.V of block 0 (tile t)
    //   E1: P of block 1 (tile t)         || QK^T of block 0 (tile t+1)
    // A block's O and l are rescaled (rarely) right after its H region: its
    // last P.V was issued in the previous region with P from before the move.
    // Carried from tile to tile: S of block 0 (tile t+1), P of block 1
    // (tile t), V^T of tile t, K fragments and K scales of tile t+1.  The copy
    // of tile t+AHEAD is spread over the E regions; past the last tile it
    // copies the last tile again into the free stage, which keeps the
    // wait counts uniform.
    using C2 = AttnCfg<DP, PV>;
    constexpr int NQK = 2 * NCB;                        // QK^T MFMAs per block and tile
    constexpr int NPV = PV == 0 ? NCB : 4 * NCB;        // P.V MFMAs
    constexpr int NRS = PV == 0 ? 1 : 4;                // row-sum MFMAs
    constexpr int NDMA = C2::NI + 1;
    v16i S[2][2];
    PHalf<PV> P[2];
    phalf_zero<PV>(P[1]);                               // P.V of block 1 for "tile -1" adds exact zeros
    v4i kf[2][NCB];
    float ksv[4];
    VA<DP, PV> va;
    if (n_main > 0 && live) {
        load_kfrag<DP>(stage_of(0).k, n, hh, kf);
        ks_of(stage_of(0), ksv);
        load_va<DP, PV>(stage_of(0).v, n, hh, va);
        qk_half<DP>(kf, qf[0], S[0]);
    }
    auto pv_region_job = [&](auto kc, const PHalf<PV>& Pj, v16f (&oj)[NCB], v4f& lsj) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k < NPV) {
            if constexpr (PV == 0) pv_job<DP, PV, k, 0>(va, Pj, oj);
            else pv_job<DP, PV, k % NCB, k / NCB>(va, Pj, oj);
        } else {
            rs_job<PV, k - NPV>(Pj, ones, lsj);
        }
    };
    for (int t = 0; t < n_main; ++t) {
        const int tc = min(t + AHEAD, ntiles - 1);      // tile copied in this step (clamped)
        const StagePtrs st_copy = stage_of(t + AHEAD);
        if (live) {
            const StagePtrs st = stage_of(t);
            const StagePtrs st_next = stage_of(t + 1);
            // H0
            SoftmaxPieces<PV> s0;
            interleave<NPV + NRS, 4>([&](auto kc) { pv_region_job(kc, P[1], o[1], ls[1]); },
                                     [&](auto hc) { s0.template head<decltype(hc)::value>(S[0], ksv, cq[0], m_ref[0],
                                                                                           m_prev[0]); });
            if (__any(s0.raise)) {
                o_guard<DP>(o[0]);
                rescale_half<DP>(m_ref[0], m_prev[0], o[0], ls[0]);
                o_guard<DP>(o[0]);
            }
            // E0
            interleave<NQK, SoftmaxPieces<PV>::NPIECE>(
                [&](auto kc) {
                    constexpr int k = decltype(kc)::value;
                    constexpr int cb = k >> 1, kb = k & 1;
                    if constexpr (cb == 0) S[1][kb] = mfma_i8_biased(kf[kb][cb], qf[1][cb]);
                    else S[1][kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kb][cb], qf[1][cb], S[1][kb], 0, 0, 0);
                    if constexpr (k == 0) load_va<DP, PV>(st.v, n, hh, va);   // V of tile t
                    if constexpr (k >= 1 && k - 1 < NDMA / 2) copier.template issue<k - 1>(st_copy, tc);
                },
                [&](auto ec) { s0.template piece<decltype(ec)::value>(S[0], P[0]); });
            // H1
            SoftmaxPieces<PV> s1;
            interleave<NPV + NRS, 4>(
                [&](auto kc) {
                    pv_region_job(kc, P[0], o[0], ls[0]);
                    if constexpr (decltype(kc)::value == 0) load_kfrag<DP>(st_next.k, n, hh, kf);   // K of tile t+1
                },
                [&](auto hc) { s1.template head<decltype(hc)::value>(S[1], ksv, cq[1], m_ref[1], m_prev[1]); });
            if (__any(s1.raise)) {
                o_guard<DP>(o[1]);
                rescale_half<DP>(m_ref[1], m_prev[1], o[1], ls[1]);
                o_guard<DP>(o[1]);
            }
            // E1
            interleave<NQK, SoftmaxPieces<PV>::NPIECE>(
                [&](auto kc) {
                    constexpr int k = decltype(kc)::value;
                    constexpr int cb = k >> 1, kb = k & 1;
                    if constexpr (cb == 0) S[0][kb] = mfma_i8_biased(kf[kb][cb], qf[0][cb]);
                    else S[0][kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kb][cb], qf[0][cb], S[0][kb], 0, 0, 0);
                    if constexpr (k >= 1 && k - 1 < NDMA - NDMA / 2) copier.template issue<NDMA / 2 + k - 1>(st_copy, tc);
                    if constexpr (k == NQK - 1) ks_of(st_next, ksv);                     // K scales of tile t+1
                },
                [&](auto ec) { s1.template piece<decltype(ec)::value>(S[1], P[1]); });
            keep_here<PV>(P[1]);
        } else {
            copier.issue_all(st_copy, tc);
        }
        wait_vmcnt<LPT * (AHEAD - 2)>();                // tile t+2 has landed
        block_sync();
    }
    if (live && n_main > 0) {                           // P.V of block 1, last pipelined tile (V is in va)
        o_guard<DP>(o[1]);                              // spaces the MFMAs from the VALU writes of P
        pv_all<DP, PV>(va, P[1], ones, o[1], ls[1]);
    }
    // the newest copy of the loop may still be in flight; the masked tiles
    // below count their own copies from zero, and the workgroup must not end
    // with a copy into its LDS outstanding
    wait_vmcnt<0>();
    int t = n_main;

    // ---- remaining tiles (a ragged end, the causal diagonal): one at a time
    for (; t < ntiles; ++t) {
        issue(t + AHEAD);
        const int k0 = t * kBK;
        if (live && (!a.causal || k0 <= wq0 + 63)) {
            const StagePtrs st = stage_of(t);
            ks_of(st, ksv);
            load_kfrag<DP>(st.k, n, hh, kf);
            qk_half<DP>(kf, qf[0], S[0]);
            qk_half<DP>(kf, qf[1], S[1]);
            const bool need_mask = (k0 + kBK > Lk) || (a.causal && k0 + kBK - 1 > wq0);
            PHalf<PV> P[2];
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
            o_guard<DP>(o[0]);
            o_guard<DP>(o[1]);
            if (__any(raised[0] || raised[1])) {
                rescale_half<DP>(m_ref[0], m_prev[0], o[0], ls[0]);
                rescale_half<DP>(m_ref[1], m_prev[1], o[1], ls[1]);
                o_guard<DP>(o[0]);
                o_guard<DP>(o[1]);
            }
            VA<DP, PV> va;
            load_va<DP, PV>(st.v, n, hh, va);
            pv_all<DP, PV>(va, P[0], ones, o[0], ls[0]);
            pv_all<DP, PV>(va, P[1], ones, o[1], ls[1]);
        }
        step_end(t);
    }
    if (!live) return;
    o_guard<DP>(o[0]);                                  // the last P.V MFMAs wrote O
    o_guard<DP>(o[1]);

    // ---- epilogue: normalise, add back V's mean, write in the caller's layout
    // the lane's channels' V scale (FP8 V only) and mean factors, all loads
    // issued before any use (the means under one uniform branch)
    const bool has_mu = a.vmean != nullptr;
    v4f sc4[NCB][4], mu4[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            if constexpr (PV == 0) sc4[cb][r4] = load_ch4(a.vs + khead * DP, cb * 32 + 8 * r4 + 4 * hh);
            mu4[cb][r4] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    if (has_mu) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) mu4[cb][r4] = load_ch4(a.vmean + khead * DP, cb * 32 + 8 * r4 + 4 * hh);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int qrow = wq0 + 32 * j + n;
        const float l_tot = ls[j][0];                   // the row-sum MFMA covers both lane halves
        const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (qrow < Lq) {
            const int64_t row_off = split * a.split_out +
                                    (a.cu_q ? (int64_t)(qoff + qrow) * a.on + (int64_t)h * a.oh
                                            : (int64_t)b * a.ob + (int64_t)h * a.oh + (int64_t)qrow * a.on);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int c0 = cb * 32 + 8 * r4 + 4 * hh;
                    if (c0 >= a.d) continue;
                    float val[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {           // channels past d are not stored
                        val[e] = o[j][cb][4 * r4 + e];
                        if constexpr (PV == 0) val[e] *= sc4[cb][r4][e] * inv_l;
                        else val[e] *= inv_l;
                        if (has_mu) val[e] += mu4[cb][r4][e];
                    }
                    store_out4<OUT_BF16>(a.out, a.out_f32, a.out_vec4, row_off, c0, a.d, val);
                }
        }
        if (a.lse) {
            constexpr float p_log2_scale = kPLog2Scale<PV>;
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
                const int64_t li = split * a.split_lse +
                                   (a.lse_varlen ? (int64_t)h * a.total_q + qoff + qrow : qhead * a.Nq + qrow);
                a.lse[li] = lse;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// FP8 P.V with two wavefronts per SIMD.  One workgroup of 8 wavefronts (two
// per SIMD) covers kBQ query rows, 32 per wavefront.  A single wavefront can
// issue a VALU instruction only every few cycles, so the softmax of one
// wavefront cannot keep pace with its own MFMAs; with two wavefronts per SIMD
// the VALU work of both runs side by side while the matrix core serves
// whichever has an MFMA ready, and each hides the other's latencies.
// Per wavefront the loop is the same software pipeline as above with one row
// block: tile t is two regions,
//   H: maximum of tile t             || P.V of tile t-1 (+ row sums)
//   E: P of tile t                   || QK^T of tile t+1
// and O is rescaled (rarely) after H.
// P.V of the 8-wavefront kernel: O^T stays in VGPRs and the MFMAs are
// compiler builtins, so the compiler sees every operand and places the wait
// states itself.
template <int DP, int CB>
__device__ __forceinline__ void pv8_job(const VA<DP, 0>& va, const PHalf<0>& P, v16f (&o)[DP / 32]) {
    o[CB] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va.a[CB], P.w, o[CB], 0, 0, 0, 0, 0, 0);
}
template <int DP>
__device__ __forceinline__ void pv8_all(const VA<DP, 0>& va, const PHalf<0>& P, const Ones<0>& ones,
                                        v16f (&o)[DP / 32], v4f& ls) {
    static_for<0, DP / 32>([&](auto cb) { pv8_job<DP, decltype(cb)::value>(va, P, o); });
    rs_job<0, 0>(P, ones, ls);
}

constexpr int kWaves8 = 8;
constexpr int kThreads8 = 64 * kWaves8;

template <int DP, bool OUT_BF16, bool KS16, bool PACK, bool QIN, bool CAUSAL>
__global__ __launch_bounds__(kThreads8, 1) void attn8_fwd_kernel(AttnArgs a) {
    constexpr int PV = 0, NW = kWaves8;                 // every wavefront copies its share
    using C = AttnCfg<DP, PV, NW, NW>;
    constexpr int NCB = C::NCB;
    constexpr int AHEAD = 5;                            // tiles in flight ahead of the one being read
    constexpr int NST = AHEAD + 3;                      // ring stages (see the key-loop comment)
    constexpr int LPT = C::NI + C::NSC;                 // copy instructions per copying wavefront per tile
    // the ring, then the epilogue's per-channel factors (V scale, V mean, K mean)
    __shared__ __attribute__((aligned(16))) uint8_t smem[NST * C::STAGE + 3 * DP * 4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hh = lane >> 5;
    const bool lead_wave = wave < kWaves8 / 2;          // wave-uniform: wavefronts 0-3 lead by half a step

    // Causal calls and varlen batches have workgroups of very different
    // lengths: those go round-robin over the XCDs (no remap) and, when causal,
    // the longest query tiles start first over the whole grid.  Other calls
    // keep the tiles of a head on one XCD, where they share its L2.
    const bool lpt = a.causal;
    int wg = (a.cu_q || a.causal) ? (int)blockIdx.x : xcd_remap(blockIdx.x, a.num_wg);
    int split = 0;
    if (a.n_splits > 1) {                               // split-KV: consecutive workgroups, consecutive key ranges
        split = wg % a.n_splits;
        wg /= a.n_splits;
    }
    const int nbh = a.num_wg / (a.n_qtiles * a.n_splits);
    int qt = lpt ? wg / nbh : wg % a.n_qtiles;
    const int bh0 = lpt ? wg % nbh : wg / a.n_qtiles, grp = a.Hq / a.Hkv;
    // Causal (longest rows first): within a row of equally long tiles, the
    // query heads of one K/V head are nkv = nbh / grp workgroups apart, so
    // that (nkv a multiple of the 8 XCDs, workgroups dealt to the XCDs in
    // turn) they share one XCD and its L2.
    const int bh = CAUSAL && grp > 1 ? (bh0 % (nbh / grp)) * grp + bh0 / (nbh / grp) : bh0;
    // packed GQA rows (non-causal, dense): the workgroup covers row r of the
    // rows of all grp query heads of one K/V head, query head
    // hk * grp + r / Nq, query r % Nq, so K and V stream once per group
    constexpr bool pack = PACK;                         // a.pack_gqa != 0
    const int b = pack ? bh / a.Hkv : bh / a.Hq;
    const int h0 = pack ? (bh % a.Hkv) * grp : bh % a.Hq;
    if (a.causal) qt = a.n_qtiles - 1 - qt;
    int Lq = a.Nq, Lk = a.Nk, qoff = 0;
    if (a.cu_q) {                                       // a sequence longer than max_seqlen is cut to it
        qoff = a.cu_q[b];
        Lq = min(max(a.cu_q[b + 1] - qoff, 0), a.Nq);
        Lk = min(max(a.cu_k[b + 1] - a.cu_k[b], 0), a.Nk);
    }
    const int kb0 = split * a.split_len;                // first key of this workgroup's range
    if (a.n_splits > 1) Lk = min(Lk - kb0, a.split_len);
    const int Lrows = pack ? grp * Lq : Lq;             // rows of the workgroup's row space
    const int q0 = qt * kBQ;
    if (q0 >= Lrows) return;
    const int hk = h0 / grp;
    const int kend = a.causal ? min(Lk, q0 + kBQ) : Lk;
    const int ntiles = (kend + kBK - 1) / kBK;
    // CAUSAL: every full tile runs in the pipelined loop, the diagonal ones
    // with the keys after each row masked; otherwise (and for the 4-wave
    // kernel) the diagonal tiles run one at a time after the loop
    const int n_main = CAUSAL ? kend / kBK : (a.causal ? min(q0, Lk) : Lk) / kBK;

    // ---- per-lane query state: row wq0 + n of the row space
    const int wq0 = q0 + wave * 32;
    const bool live = wq0 < Lrows;
    int h, qrow;
    bool lane_ok;
    if (pack) {
        const int r = wq0 + n;
        lane_ok = r < Lrows;
        const int hi = lane_ok ? r / Lq : 0;
        h = h0 + hi;
        qrow = lane_ok ? r - hi * Lq : 0;
    } else {
        h = h0;
        qrow = wq0 + n;
        lane_ok = qrow < Lq;
    }
    const int64_t qhead = (int64_t)b * a.Hq + h;
    v4i qf[NCB];
    float qscale = 0.f;
    // With Q in its input precision (QIN) the lane loads the 8-channel slices
    // cb*32 + hh*16 + 8e of its row here and quantizes them after the
    // prologue's copies are issued (rows past the sequence load its first row
    // and slices past d the first slice; both become zeros).
    v4i qraw[2 * NCB];
    if constexpr (QIN) {
        const int qr = lane_ok ? qrow : 0;
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.qraw) +
                             (a.cu_q ? (int64_t)(qoff + qr) * a.qsn + (int64_t)h * a.qsh
                                     : (int64_t)b * a.qsb + (int64_t)h * a.qsh + (int64_t)qr * a.qsn);
#pragma unroll
        for (int i = 0; i < 2 * NCB; ++i) {
            const int c0 = (i >> 1) * 32 + hh * 16 + 8 * (i & 1);
            qraw[i] = *reinterpret_cast<const v4i*>(qp + (c0 < a.d ? c0 : 0));
        }
    } else if (live) {
        const int8_t* q8row = a.q8 + (qhead * a.nq_pad + qrow) * DP;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) qf[cb] = *reinterpret_cast<const v4i*>(q8row + cb * 32 + hh * 16);
        qscale = a.qs[qhead * (a.nq_pad >> a.gq_shift) + (qrow >> a.gq_shift)];
    } else {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) qf[cb] = v4i{0, 0, 0, 0};
    }
    float cq = 0.f;                                     // log2-domain row factor times 2^26 (exact)
    if constexpr (!QIN) cq = ((qscale * a.sm_scale) * kLog2e) * kAccScale;

    const int64_t khead = (int64_t)b * a.Hkv + hk;
    // The epilogue's per-channel factors of this K/V head (V scale, V mean, K
    // mean; V's scale row stands in for an absent mean) are loaded here and
    // staged in LDS past the ring after the prologue's barrier: every lane
    // needs 64 of them, and 512 threads reading them from L2 at the end took
    // microseconds.
    constexpr int FPL = DP / 64;                        // factors per lane per row
    float fac[3][FPL];
    {
        const float* fs = a.vs + khead * DP;
        const float* fm = a.vmean ? a.vmean + khead * DP : fs;
        const float* fk = a.kmean ? a.kmean + khead * DP : fs;
#pragma unroll
        for (int j = 0; j < FPL; ++j) {
            fac[0][j] = fs[lane * FPL + j];
            fac[1][j] = fm[lane * FPL + j];
            fac[2][j] = fk[lane * FPL + j];
        }
    }
    const int8_t* kbase = uniform(a.k8 + khead * a.nk_pad * DP + (int64_t)kb0 * DP);
    const float* ksbase = uniform(a.ks + khead * (a.nk_pad >> a.gk_shift) + (kb0 >> a.gk_shift));
    const uint8_t* vbase = uniform(reinterpret_cast<const uint8_t*>(a.vt) + khead * DP * a.nk_pad + kb0);
    const int64_t vrow_stride = a.nk_pad;
    const bool ks16 = a.gk_shift == 4;

    v16f o[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cb][i] = 0.f;
    v4f ls = v4f{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, m_prev;
    Ones<PV> ones;
    make_ones<PV>(ones, rowsum_parity(lane));

    auto stage_of = [&](int t) { return ring_stage<C, NST>(smem, t % NST); };
    auto ks_of = [&](const StagePtrs& st, float (&ksv)[4]) {
        const v4f k4 = *reinterpret_cast<const v4f*>(st.s + wave * 256);
#pragma unroll
        for (int g = 0; g < 4; ++g) ksv[g] = k4[g];
    };
    // This lane's LDS addresses in ring stage 0, held in registers for the
    // whole loop: the K fragments of each channel block, the two 16-byte
    // halves of its V^T operand, and its wavefront's K-scale slot.  A read of
    // stage u in the pipelined loop adds only a constant below 64 KB (u times
    // the region's bytes per stage, plus the key or channel block), which the
    // LDS instruction takes as its immediate offset.  The empty asm statements
    // keep the compiler from recombining the bases with those constants, which
    // costs an add per read.
    typedef __attribute__((address_space(3))) const uint8_t lds_u8;
    typedef __attribute__((address_space(3))) const v4i lds_v4i;
    typedef __attribute__((address_space(3))) const v4f lds_v4f;
    lds_u8* kp[NCB];
    lds_u8* vp[2];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        kp[cb] = (lds_u8*)(smem + n * DP + swz<DP>(n, cb * 2 + hh) * 16);
        asm volatile("" : "+v"(kp[cb]));
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        vp[e] = (lds_u8*)(smem + NST * C::KT_BYTES + n * C::VROW + swz<C::VROW>(n, 2 * hh + e) * 16);
        asm volatile("" : "+v"(vp[e]));
    }
    lds_u8* sp_slot = (lds_u8*)(smem + NST * (C::KT_BYTES + C::VT_BYTES) + wave * 256);
    asm volatile("" : "+v"(sp_slot));
    const TileCopyBuf<DP, PV, NW, NW> copier(kbase, vbase, (uint32_t)vrow_stride, ksbase,
                                                  (uint32_t)(a.nk_pad - kb0) * DP, (uint32_t)(a.nk_pad * DP - kb0),
                                                  (uint32_t)((a.nk_pad - kb0) >> a.gk_shift) * 4u, ks16, wave, lane);
    auto issue = [&](int t) {
        if (t < ntiles) copier.issue_all(stage_of(t), t);
    };
    auto step_end = [&](int t) {
        if (t + AHEAD < ntiles) wait_vmcnt<LPT * (AHEAD - 2)>();
        else wait_vmcnt<0>();
        block_sync();
    };

    // prologue: tiles 0 .. AHEAD-1 in flight, tiles 0 .. 2 landed.  The
    // copies are unconditional (past the last tile they copy it again, into
    // stages no step reads), so that the number of loads in flight is the
    // same on every path and the compiler waits for the Q fragments without
    // waiting for the whole prologue.
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) copier.issue_all(stage_of(u), max(min(u, ntiles - 1), 0));

    // Q in its input precision -> INT8 codes and scales, as the quantize pass
    // makes them: the absolute maximum of the row (its two lanes), of the
    // wavefront's 32 rows (per_warp), or of 4 wavefronts' 128 rows through
    // LDS (per_block).  The raw values pass through an empty asm statement
    // first, so that no part of their unpacking is moved above the copies
    // (which would wait for the Q loads before the copies are issued).  The
    // LDS slots are the first bytes of the ring's last stage, which no copy
    // fills before step 2, when every wavefront has long read them (a
    // separate LDS array would keep the compiler from telling the ring's
    // reads apart from its copies, and it would then wait for every copy in
    // flight before each read).
    float* s_qmax = reinterpret_cast<float*>(smem + (NST - 1) * C::KT_BYTES);
    float qx[2 * NCB][8];
    float qm = 0.f;
    if constexpr (QIN) {
#pragma unroll
        for (int i = 0; i < 2 * NCB; ++i) asm volatile("" : "+v"(qraw[i]));
#pragma unroll
        for (int i = 0; i < 2 * NCB; ++i) {           // rows past the sequence and slices past d: zeros
            const bool ok = lane_ok && (i >> 1) * 32 + hh * 16 + 8 * (i & 1) < a.d;
            qraw[i] = ok ? qraw[i] : v4i{0, 0, 0, 0};
        }
        if (a.q_bf16) {
#pragma unroll
            for (int i = 0; i < 2 * NCB; ++i) unpack8<true>(__builtin_bit_cast(uint4, qraw[i]), qx[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 2 * NCB; ++i) unpack8<false>(__builtin_bit_cast(uint4, qraw[i]), qx[i]);
        }
#pragma unroll
        for (int i = 0; i < 2 * NCB; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) qm = fmaxf(qm, fabsf(qx[i][j]));
        qm = fmaxf(qm, __shfl_xor(qm, 32));
        if (a.gq_shift >= 5) {
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) qm = fmaxf(qm, __shfl_xor(qm, off));
        }
        if (a.gq_shift == 7 && lane == 0) s_qmax[wave] = qm;
        wait_lgkm0();
    }
    wait_vmcnt<LPT * (AHEAD - 3)>();
    block_sync();
    if constexpr (QIN) {
        if (a.gq_shift == 7) {
            const int w0 = wave & ~3;
            qm = fmaxf(fmaxf(s_qmax[w0], s_qmax[w0 + 1]), fmaxf(s_qmax[w0 + 2], s_qmax[w0 + 3]));
        }
        float inv;
        int8_group_scale(qm, qscale, inv);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const uint2 lo = int8_codes8(qx[2 * cb], inv), hi = int8_codes8(qx[2 * cb + 1], inv);
            qf[cb] = v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
        }
        cq = ((qscale * a.sm_scale) * kLog2e) * kAccScale;
    }
    float* s_fac = reinterpret_cast<float*>(smem + NST * C::STAGE);
    if (wave == 0) {                                    // read in the epilogue, after many barriers
#pragma unroll
        for (int f = 0; f < 3; ++f)
#pragma unroll
            for (int j = 0; j < FPL; ++j) s_fac[f * DP + lane * FPL + j] = fac[f][j];
        wait_lgkm0();
    }

    constexpr int NQK = 2 * NCB;
    constexpr int NPV = NCB;
    constexpr int NRS = 1;
    constexpr int NDMA = LPT;
    // Step t is two regions:
    //   H(t): QK^T of tile t, then P.V of tile t-1 and the row sums, with the
    //         group maxima of tile t and the raise decision (the new
    //         reference maximum of every row) between the P.V MFMAs, the copy
    //         of tile t+AHEAD, and the K and V^T fragments of the next step
    //         (matrix-core work);
    //   E(t): P of tile t against the new maximum; then, if some row of the
    //         wavefront moved its maximum, O and the row sums (complete up to
    //         tile t-1 by now) are rescaled (VALU work).
    // One workgroup barrier per step: wavefronts 0-3 pass barrier t right
    // after their H(t), wavefronts 4-7 right before theirs, so between
    // barriers t and t+1 the leading group runs E(t) then H(t+1) while the
    // other runs H(t) then E(t), and on each SIMD one wavefront is mostly in
    // H while the other is in E.  The ring stays valid with NST = AHEAD + 3
    // stages when every wavefront waits for its own share of tile t+3 at the
    // end of its H(t):
    //  * reads of tile t+1 (K fragments in H(t)) come after barrier t-1 for
    //    the leading group and after barrier t for the other; every share of
    //    tile t+1 was waited for in an H(t-2), which both groups finish
    //    before barrier t-1;
    //  * the copy in H(t) overwrites the stage of tile t+AHEAD-NST = t-3,
    //    whose last fragment reads (V^T in H(t-3), consumed by the MFMAs of
    //    H(t-2)) both groups finish before barrier t-1, which precedes H(t)
    //    of either group.
    v16i S[2];
    PHalf<PV> P;
    phalf_zero<PV>(P);                                  // P.V for "tile -1" adds exact zeros
    v4i kf[2][NCB];
    float ksv[4];
    VA<DP, PV> va;
    if (n_main > 0 && live) {
        load_kfrag<DP>(stage_of(0).k, n, hh, kf);
        ks_of(stage_of(0), ksv);
        load_va<DP, PV>(stage_of(0).v, n, hh, va);
    }
    constexpr int NH = NQK + NPV + NRS;                 // matrix-core jobs of H
    static_assert(NPV + NRS >= 3, "room for the group maxima");
    // u = t % NST as a compile-time constant: every LDS address of the step
    // is a fixed offset from one base
    auto regionH = [&](auto u, int t, SoftmaxPieces<PV, KS16>& sp) {
        constexpr int U = decltype(u)::value;
        const int tc = min(t + AHEAD, ntiles - 1);
        constexpr int UN = (U + 1) % NST;               // stage of tile t+1
        const StagePtrs st_copy = ring_stage<C, NST>(smem, (U + AHEAD) % NST);
        if (live) {
            static_for<0, NH>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if constexpr (k < NQK) {
                    constexpr int kb = k & 1, cb = k >> 1;
                    if constexpr (cb == 0) S[kb] = mfma_i8_biased(kf[kb][cb], qf[cb]);
                    else S[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kb][cb], qf[cb], S[kb], 0, 0, 0);
                } else if constexpr (k < NQK + NPV) {
                    pv8_job<DP, k - NQK>(va, P, o);
                } else {
                    rs_job<PV, 0>(P, ones, ls);
                }
                if constexpr (k >= 1 && k - 1 < NDMA) copier.template issue<k - 1>(st_copy, tc);
                if constexpr (k == 0) {
                    sp.prep(ksv, cq);
                    if constexpr (CAUSAL) sp.floor_f();
                }
                if constexpr (k == NQK - 1) {           // K of tile t+1 (kf is free once the last QK^T MFMA issued)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
                            kf[kb][cb] = *(lds_v4i*)(kp[cb] + UN * C::KT_BYTES + kb * 32 * DP);
                }
                // group maxima of tile t, one or two per P.V MFMA, then the
                // raise decision
                // a tile with keys after the wavefront's first row: the
                // scores of keys after the lane's row become the -inf pattern
                if constexpr (CAUSAL && (k == NQK + 1 || k == NQK + 2)) {
                    constexpr int kb = k - NQK - 1;
                    if (t * kBK + kBK - 1 > wq0) causal_mask_half(S[kb], qrow - t * kBK - kb * 32 - 4 * hh);
                }
                if constexpr (k == NQK + 1) { sp.gmax(S[0], 0); sp.gmax(S[0], 1); }
                if constexpr (k == NQK + 2) { sp.gmax(S[1], 2); sp.gmax(S[1], 3); }
                if constexpr (k == NH - 1) sp.decide(m_ref, m_prev);
                if constexpr (k == NH - 1) {            // V of tile t (va is free once the last P.V MFMA issued)
                    const v4f k4 = *(lds_v4f*)(sp_slot + UN * C::SC_BYTES);
#pragma unroll
                    for (int g = 0; g < 4; ++g) ksv[g] = k4[g];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const int off = U * C::VT_BYTES + cb * 32 * C::VROW;
                        const v4i lo = *(lds_v4i*)(vp[0] + off), hi = *(lds_v4i*)(vp[1] + off);
                        va.a[cb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    }
                }
                sched_fence();
            });
        } else {
            copier.issue_all(st_copy, tc);
        }
        wait_vmcnt<LPT * (AHEAD - 3)>();                // own share of tile t+3 has landed
    };
    auto regionE = [&](SoftmaxPieces<PV, KS16>& sp) {
        if (!live) return;
        sp.spec(m_ref);
        static_for<0, SoftmaxPieces<PV, KS16>::NPIECE>([&](auto ec) { sp.template piece<decltype(ec)::value>(S, P); });
        keep_here<PV>(P);
        if (__any(sp.raise)) rescale_half<DP>(m_ref, m_prev, o, ls);   // some row moved its maximum
    };
    // both groups pass one barrier per step (see above); a last barrier
    // after the loop orders every wavefront's final waits before the tail
    auto step = [&](auto u, int t) {
        SoftmaxPieces<PV, KS16> sp;
        if (!lead_wave) block_sync();
        regionH(u, t, sp);
        if (lead_wave) block_sync();
        regionE(sp);
    };
    int t = 0;
    for (; t < n_main; t += NST) {                      // stage slots 0 .. NST-1 in turn
        static_for<0, NST>([&](auto u) {
            if (t + decltype(u)::value < n_main) step(u, t + decltype(u)::value);
        });
    }
    t = n_main;
    if (live && n_main > 0) pv8_all<DP>(va, P, ones, o, ls);   // P.V of the last pipelined tile
    wait_vmcnt<0>();
    block_sync();

    // ---- remaining tiles (a ragged end, the causal diagonal): one at a time
    for (; t < ntiles; ++t) {
        issue(t + AHEAD);
        const int k0 = t * kBK;
        if (live && (!a.causal || k0 <= wq0 + 31)) {
            const StagePtrs st = stage_of(t);
            ks_of(st, ksv);
            load_kfrag<DP>(st.k, n, hh, kf);
            v16i Sm[2];
                qk_half<DP>(kf, qf, Sm);
            const bool need_mask = (k0 + kBK > Lk) || (a.causal && k0 + kBK - 1 > wq0);
            PHalf<PV> Pm;
            bool raised;
            if (need_mask)
                raised = softmax_half<PV, true>(Sm, ksv, cq, m_ref, m_prev, Pm, k0, Lk, a.causal, qrow, hh);
            else
                raised = softmax_half<PV, false>(Sm, ksv, cq, m_ref, m_prev, Pm, k0, Lk, a.causal, qrow, hh);
            if (__any(raised)) rescale_half<DP>(m_ref, m_prev, o, ls);
            VA<DP, PV> vam;
            load_va<DP, PV>(st.v, n, hh, vam);
            pv8_all<DP>(vam, Pm, ones, o, ls);
        }
        step_end(t);
    }
    if (!live) return;

    // ---- epilogue: normalise, add back V's mean, write in the caller's layout,
    // with the lane's channels' V scale and mean factors from LDS
    const bool has_mu = a.vmean != nullptr;
    v4f sc4[NCB][4], mu4[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int c0 = cb * 32 + 8 * r4 + 4 * hh;
            sc4[cb][r4] = *(lds_v4f*)(s_fac + c0);
            mu4[cb][r4] = *(lds_v4f*)(s_fac + DP + c0);
        }
    const float l_tot = ls[0];
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    auto out_val = [&](int cb, int r4, float (&val)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            val[e] = o[cb][4 * r4 + e] * (sc4[cb][r4][e] * inv_l);
            if (has_mu) val[e] += mu4[cb][r4][e];
        }
    };
    if (a.out_vec8) {
        // 16-bit rows with 16-byte alignment: the wavefront stages its 32 rows
        // in its own slice of the ring (free now: every copy has landed and
        // every wavefront has passed the last barrier), rows padded by 16 bytes
        // against bank conflicts, then stores whole 16-byte pieces, 64 of
        // them per instruction over consecutive row memory.  (Straight from
        // the MFMA layout, each store instruction wrote 8 bytes into each of
        // 32 rows, and the stores took about half of the epilogue.)
        constexpr int RS = DP * 2 + 16;                 // bytes per staged row
        constexpr int CPR = DP / 8;                     // 16-byte pieces per row
        uint8_t* wt = smem + wave * 32 * RS;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float val[4];
                out_val(cb, r4, val);
                uint16_t hv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = Half<OUT_BF16>::from_f(val[e]);
                *reinterpret_cast<uint2*>(wt + n * RS + (cb * 32 + 8 * r4 + 4 * hh) * 2) =
                    make_uint2((uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16));
            }
        wait_lgkm0();                                   // the wavefront reads back only its own rows
#pragma unroll
        for (int i = 0; i < 32 * CPR / 64; ++i) {
            const int q = i * 64 + lane, r = q / CPR, c8 = (q % CPR) * 8;
            const int rr = wq0 + r;                     // row of the workgroup's row space
            if (rr >= Lrows || c8 >= a.d) continue;
            int hr = h0, qr = rr;
            if (pack) {
                const int hi = rr / Lq;
                hr = h0 + hi;
                qr = rr - hi * Lq;
            }
            const int64_t row_off = split * a.split_out +
                                    (a.cu_q ? (int64_t)(qoff + qr) * a.on + (int64_t)hr * a.oh
                                            : (int64_t)b * a.ob + (int64_t)hr * a.oh + (int64_t)qr * a.on);
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + row_off + c8) =
                *reinterpret_cast<const uint4*>(wt + r * RS + c8 * 2);
        }
    } else if (lane_ok) {
        const int64_t row_off = split * a.split_out +
                                (a.cu_q ? (int64_t)(qoff + qrow) * a.on + (int64_t)h * a.oh
                                        : (int64_t)b * a.ob + (int64_t)h * a.oh + (int64_t)qrow * a.on);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int c0 = cb * 32 + 8 * r4 + 4 * hh;
                if (c0 >= a.d) continue;                // channels past d are not stored
                float val[4];
                out_val(cb, r4, val);
                store_out4<OUT_BF16>(a.out, a.out_f32, a.out_vec4, row_off, c0, a.d, val);
            }
    }
    if (a.lse) {
        constexpr float p_log2_scale = kPLog2Scale<0>;
        float part = 0.f;
        if (a.kmean) {
            v4f km4[NCB][4];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int u = 0; u < 4; ++u) km4[cb][u] = *(lds_v4f*)(s_fac + 2 * DP + cb * 32 + hh * 16 + 4 * u);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int code = (int)(int8_t)((qf[cb][e >> 2] >> (8 * (e & 3))) & 0xff);
                    part += (float)code * km4[cb][e >> 2][e & 3];
                }
        }
        const float dot = swap_half_sum(part);
        if (hh == 0 && lane_ok) {
            const float corr = a.kmean ? a.sm_scale * qscale * dot : 0.f;
            const float lse = (m_ref + __log2f(l_tot) - p_log2_scale) * kLn2 + corr;
            const int64_t li = split * a.split_lse +
                               (a.lse_varlen ? (int64_t)h * a.total_q + qoff + qrow : qhead * a.Nq + qrow);
            a.lse[li] = lse;
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
    int Lq = a.Nq, Lk = a.Nk, qoff = 0;                 // varlen: this sequence's lengths (as the forward cuts them)
    if (a.cu_q) {
        qoff = a.cu_q[b];
        Lq = min(max(a.cu_q[b + 1] - qoff, 0), a.Nq);
        Lk = min(max(a.cu_k[b + 1] - a.cu_k[b], 0), a.Nk);
    }
    const int64_t qhead = (int64_t)b * a.Hq + h;
    const int8_t* q8row = a.q8 + (qhead * a.nq_pad + qrow) * DP;
    // the same fragment code as the attention kernel, with both row blocks
    // holding this wavefront's 32 rows
    v4i qf[2][DP / 32];
#pragma unroll
    for (int cb = 0; cb < DP / 32; ++cb)
        qf[0][cb] = qf[1][cb] = *reinterpret_cast<const v4i*>(q8row + cb * 32 + hh * 16);
    const int8_t* kbase = a.k8 + ((int64_t)b * a.Hkv + hk) * a.nk_pad * DP;
    const int ntiles = (Lk + kBK - 1) / kBK;
    unsigned long long s1 = 0, s2 = 0;
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
        qk_half<DP>(kf, qf[0], acc[0]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = t * kBK + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
                const int S = acc[0][kb][i] - kAccBiasBits;
                if (key < Lk) {
                    if (a.dbg_mode == 0) {
                        if (qrow < Lq)
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
        if (hh == 0 && qrow < Lq) {
            const int64_t row = a.cu_q ? (int64_t)h * a.total_q + qoff + qrow : qhead * a.Nq + qrow;
            unsigned long long* d = reinterpret_cast<unsigned long long*>(a.dbg) + row * 2;
            d[0] = s1;
            d[1] = s2;
        }
    }
}

// ---------------------------------------------------------------------------
// The 8-wavefront kernel with INT8 Q, or (128 channels) the one that
// quantizes Q itself; the host accepts Q in its input precision only there.
template <int DP, bool OUT_BF16, bool KS16, bool PACK, bool QIN>
static void launch8c(const AttnArgs& a, hipStream_t s) {
    if constexpr (!PACK) {                              // packed rows are non-causal only
        if (a.causal) {
            attn8_fwd_kernel<DP, OUT_BF16, KS16, PACK, QIN, true><<<a.num_wg, kThreads8, 0, s>>>(a);
            return;
        }
    }
    attn8_fwd_kernel<DP, OUT_BF16, KS16, PACK, QIN, false><<<a.num_wg, kThreads8, 0, s>>>(a);
}

template <int DP, bool OUT_BF16, bool KS16, bool PACK>
static void launch8(const AttnArgs& a, hipStream_t s) {
    if constexpr (DP == 128) {
        if (a.qraw) {
            launch8c<DP, OUT_BF16, KS16, PACK, true>(a, s);
            return;
        }
    }
    launch8c<DP, OUT_BF16, KS16, PACK, false>(a, s);
}

template <int DP, int PV>
static void attn_dispatch_out(const AttnArgs& a, bool out_bf16, hipStream_t s) {
    if constexpr (PV == 0) {
        const bool ks16 = a.gk_shift == 4;              // per_thread K groups of 16 keys
        if (a.pack_gqa) {
            if (out_bf16) {
                if (ks16) launch8<DP, true, true, true>(a, s);
                else launch8<DP, true, false, true>(a, s);
            } else {
                if (ks16) launch8<DP, false, true, true>(a, s);
                else launch8<DP, false, false, true>(a, s);
            }
        } else if (out_bf16) {
            if (ks16) launch8<DP, true, true, false>(a, s);
            else launch8<DP, true, false, false>(a, s);
        } else {
            if (ks16) launch8<DP, false, true, false>(a, s);
            else launch8<DP, false, false, false>(a, s);
        }
    } else {
        if (out_bf16) attn_fwd_kernel<DP, PV, true><<<a.num_wg, kThreads, 0, s>>>(a);
        else attn_fwd_kernel<DP, PV, false><<<a.num_wg, kThreads, 0, s>>>(a);
    }
}

hipError_t launch_attn(const AttnArgs& a_in, int dp, int pv, bool out_bf16, hipStream_t s) {
    AttnArgs a = a_in;
    const int grp = a.Hq / a.Hkv;
    a.n_qtiles = ((a.pack_gqa ? grp : 1) * a.Nq + kBQ - 1) / kBQ;
    if (a.n_splits < 1) a.n_splits = 1;
    a.num_wg = a.B * (a.pack_gqa ? a.Hkv : a.Hq) * a.n_qtiles * a.n_splits;
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
