// sage_api.hip -- the C ABI (include/sage.h): argument validation on the
// host, workspace layout, and the launch sequence of each entry point.
//
// Every entry point validates all of its arguments before the first HIP call,
// so an invalid call launches nothing and writes nothing; errors are reported
// as a status code plus a thread-local message (sage_last_error()).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "sage.h"
#include "sage_kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return SAGE_OK;
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }
int dp_of(int d) { return d <= 64 ? 64 : 128; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int q_group_shift(int gran) { return gran == SAGE_PER_BLOCK ? 7 : gran == SAGE_PER_WARP ? 5 : 0; }
int k_group_shift(int gran) { return gran == SAGE_PER_THREAD ? 4 : 6; }
bool valid_gran(int g) { return g == SAGE_PER_BLOCK || g == SAGE_PER_WARP || g == SAGE_PER_THREAD; }
bool valid_dtype(int t) { return t == SAGE_F16 || t == SAGE_BF16; }

constexpr int64_t kMaxDim = 1 << 30;

int check_sizes(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1)
        return fail(SAGE_EINVAL, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d)", B, Hq, Hkv, Nq, Nk);
    if (d < 1 || d > 128) return fail(SAGE_EINVAL, "head_dim %d unsupported: must be 1..128", d);
    if (Hq % Hkv != 0) return fail(SAGE_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if ((int64_t)B * Hq > kMaxDim || Nq > kMaxDim - 256 || Nk > kMaxDim - 256)
        return fail(SAGE_EINVAL, "sizes too large");
    return SAGE_OK;
}

struct WsLayout {
    size_t sum_off, min_off, max_off, total;
    int chunk_len;
    int chunks;
};

WsLayout ws_layout(int B, int H, int N, int d) {
    WsLayout w{};
    const int dp = dp_of(d);
    // kStatsChunk tokens per chunk, longer (a multiple of it) beyond the target
    // number of chunks per (sequence, head): about 256 statistics workgroups in
    // all, 8 to kMaxChunks per head.  Fewer chunks mean fewer partials for
    // every tile workgroup of the second pass to reduce; enough of them keep
    // the statistics pass spread over the GPU.
    const int64_t heads = (int64_t)B * H;
    const int64_t target = std::min<int64_t>(sage::kMaxChunks, std::max<int64_t>(8, (256 + heads - 1) / heads));
    const int64_t per = (N + target - 1) / target;
    w.chunk_len = (int)std::max<int64_t>(sage::kStatsChunk, round_up(per, sage::kStatsChunk));
    w.chunks = (int)((N + w.chunk_len - 1) / w.chunk_len);
    const size_t cells = (size_t)B * H * w.chunks * dp;
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    w.sum_off = 0;
    w.min_off = al(cells * 8);
    w.max_off = w.min_off + al(cells * 4);
    w.total = w.max_off + al(cells * 4);
    return w;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SAGE_EHIP, "%s: %s", what, hipGetErrorString(e));
    return SAGE_OK;
}

}  // namespace

extern "C" {

const char* sage_last_error(void) { return g_err.c_str(); }
int sage_version(void) { return SAGE_ABI_VERSION; }

size_t sage_quant_workspace_size(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1 || d < 1 || d > 128) return 0;
    return ws_layout(B, H, N, d).total;
}

namespace {
// Validated launch arguments of one quantize call.
struct QKPrep {
    sage::QuantRowsArgs qa, ka;
    sage::StatsArgs st;
    bool smooth, bf16, vec;
    WsLayout wl;
    const void* ws;
    size_t ws_used;                     // bytes of workspace the call uses (0: none)
};
struct VPrep {
    sage::QuantVArgs va;
    sage::StatsArgs st;
    bool need_stats, smooth, bf16, fp8, vec;
    WsLayout wl;
    const void* ws;
    size_t ws_used;
};

// Point the statistics partials of a prepared call at workspace `base`
// (NULL: no workspace bound yet).
void bind_qk_ws(QKPrep& o, uint8_t* base) {
    o.ws = o.ws_used ? base : nullptr;
    if (o.smooth) o.st.part_sum = base ? base + o.wl.sum_off : nullptr;
}
void bind_v_ws(VPrep& o, uint8_t* base) {
    o.ws = o.ws_used ? base : nullptr;
    if (o.need_stats) {
        o.st.part_sum = base ? base + o.wl.sum_off : nullptr;
        o.st.part_min = base ? reinterpret_cast<float*>(base + o.wl.min_off) : nullptr;
        o.st.part_max = base ? reinterpret_cast<float*>(base + o.wl.max_off) : nullptr;
    }
}

// Validate a Q/K quantize call and build its launch arguments.  With
// own_ws = false the caller's workspace fields are ignored (and not checked);
// the partials are bound later with bind_qk_ws.
int prepare_qk(const sage_quant_qk_params* p, QKPrep& o, bool own_ws = true) {
    if (!p) return fail(SAGE_EINVAL, "params is NULL");
    if (p->struct_size < sizeof(sage_quant_qk_params)) return fail(SAGE_EINVAL, "struct_size too small");
    if (!valid_dtype(p->dtype)) return fail(SAGE_EINVAL, "unknown dtype %d", p->dtype);
    if (int r = check_sizes(p->B, p->Hq, p->Hkv, p->Nq, p->Nk, p->d)) return r;
    if (!valid_gran(p->gran)) return fail(SAGE_EINVAL, "unknown qk_quant_gran %d", p->gran);
    const bool with_q = p->q || p->q8 || p->q_scale;    // all three NULL: K only
    if ((with_q && (!p->q || !p->q8 || !p->q_scale)) || !p->k || !p->k8 || !p->k_scale)
        return fail(SAGE_EINVAL, "NULL tensor pointer");
    if (p->smooth_k && !p->k_mean) return fail(SAGE_EINVAL, "smooth_k needs k_mean");
    if (!aligned(p->q, 2) || !aligned(p->k, 2)) return fail(SAGE_EINVAL, "q/k not 2-byte aligned");   // (NULL is aligned)
    if (!aligned(p->q8, 16) || !aligned(p->k8, 16)) return fail(SAGE_EINVAL, "q8/k8 must be 16-byte aligned");
    if (!aligned(p->q_scale, 4) || !aligned(p->k_scale, 4) || (p->k_mean && !aligned(p->k_mean, 4)))
        return fail(SAGE_EINVAL, "scales/means must be 4-byte aligned");
    if ((p->cu_seqlens_q == nullptr) != (p->cu_seqlens_k == nullptr))
        return fail(SAGE_EINVAL, "cu_seqlens_q and cu_seqlens_k must both be given or both be NULL");
    if (p->q_stride_n <= 0 || p->k_stride_n <= 0 || p->q_stride_h < 0 || p->k_stride_h < 0 ||
        p->q_stride_b < 0 || p->k_stride_b < 0)
        return fail(SAGE_EINVAL, "negative or zero token stride");
    const WsLayout ws = ws_layout(p->B, p->Hkv, p->Nk, p->d);
    if (p->smooth_k && own_ws) {
        if (!p->workspace || !aligned(p->workspace, 16)) return fail(SAGE_EINVAL, "workspace NULL or misaligned");
        if (p->workspace_bytes < ws.total)
            return fail(SAGE_EINVAL, "workspace too small: %zu < %zu bytes", p->workspace_bytes, ws.total);
    }
    const bool bf16 = p->dtype == SAGE_BF16;
    const int dp = dp_of(p->d);
    const int nq_pad = (int)round_up(p->Nq, sage::kPad), nk_pad = (int)round_up(p->Nk, sage::kPad);
    sage::StatsArgs st{};
    st.x = p->k; st.sb = p->k_stride_b; st.sh = p->k_stride_h; st.sn = p->k_stride_n;
    st.cu = p->cu_seqlens_k; st.B = p->B; st.H = p->Hkv; st.N = p->Nk; st.d = p->d; st.dp = dp;
    st.chunks = ws.chunks; st.chunk_len = ws.chunk_len; st.want_minmax = 0;
    if (p->smooth_k) st.out_mean = p->k_mean;
    auto vec_ok = [&](const void* x, int64_t sb, int64_t sh, int64_t sn) {
        return aligned(x, 16) && p->d % 8 == 0 && sb % 8 == 0 && sh % 8 == 0 && sn % 8 == 0;
    };
    sage::QuantRowsArgs qa{};
    qa.x = p->q; qa.sb = p->q_stride_b; qa.sh = p->q_stride_h; qa.sn = p->q_stride_n; qa.cu = p->cu_seqlens_q;
    qa.B = p->B; qa.H = p->Hq; qa.N = p->Nq; qa.npad = nq_pad; qa.d = p->d;
    qa.group_shift = q_group_shift(p->gran); qa.out = p->q8; qa.scale = p->q_scale;
    sage::QuantRowsArgs ka{};
    ka.x = p->k; ka.sb = p->k_stride_b; ka.sh = p->k_stride_h; ka.sn = p->k_stride_n; ka.cu = p->cu_seqlens_k;
    ka.B = p->B; ka.H = p->Hkv; ka.N = p->Nk; ka.npad = nk_pad; ka.d = p->d;
    ka.group_shift = k_group_shift(p->gran); ka.out = p->k8; ka.scale = p->k_scale;
    const bool vec = (!with_q || vec_ok(p->q, p->q_stride_b, p->q_stride_h, p->q_stride_n)) &&
                     vec_ok(p->k, p->k_stride_b, p->k_stride_h, p->k_stride_n);
    o.qa = qa;
    o.ka = ka;
    o.st = st;
    o.smooth = p->smooth_k != 0;
    o.bf16 = bf16;
    o.vec = vec;
    o.wl = ws;
    o.ws_used = p->smooth_k ? ws.total : 0;
    bind_qk_ws(o, own_ws ? reinterpret_cast<uint8_t*>(p->workspace) : nullptr);
    return 0;
}

// As prepare_qk, for a V quantize call.
int prepare_v(const sage_quant_v_params* p, VPrep& o, bool own_ws = true) {
    if (!p) return fail(SAGE_EINVAL, "params is NULL");
    if (p->struct_size < sizeof(sage_quant_v_params)) return fail(SAGE_EINVAL, "struct_size too small");
    if (!valid_dtype(p->dtype)) return fail(SAGE_EINVAL, "unknown dtype %d", p->dtype);
    if (int r = check_sizes(p->B, p->Hkv, p->Hkv, p->Nk, p->Nk, p->d)) return r;
    if (p->v_dtype != SAGE_V_FP8 && p->v_dtype != SAGE_V_FP16) return fail(SAGE_EINVAL, "unknown v_dtype %d", p->v_dtype);
    const bool fp8 = p->v_dtype == SAGE_V_FP8;
    if (!p->v || !p->vt) return fail(SAGE_EINVAL, "NULL tensor pointer");
    if (fp8 && !p->v_scale) return fail(SAGE_EINVAL, "FP8 V needs v_scale");
    if (p->smooth_v && !p->v_mean) return fail(SAGE_EINVAL, "smooth_v needs v_mean");
    if (!aligned(p->v, 2)) return fail(SAGE_EINVAL, "v not 2-byte aligned");
    if (!aligned(p->vt, 16)) return fail(SAGE_EINVAL, "vt must be 16-byte aligned");
    if ((p->v_scale && !aligned(p->v_scale, 4)) || (p->v_mean && !aligned(p->v_mean, 4)))
        return fail(SAGE_EINVAL, "scales/means must be 4-byte aligned");
    if (p->v_stride_n <= 0 || p->v_stride_h < 0 || p->v_stride_b < 0)
        return fail(SAGE_EINVAL, "negative or zero token stride");
    const bool need_stats = fp8 || p->smooth_v;
    const WsLayout ws = ws_layout(p->B, p->Hkv, p->Nk, p->d);
    if (need_stats && own_ws) {
        if (!p->workspace || !aligned(p->workspace, 16)) return fail(SAGE_EINVAL, "workspace NULL or misaligned");
        if (p->workspace_bytes < ws.total)
            return fail(SAGE_EINVAL, "workspace too small: %zu < %zu bytes", p->workspace_bytes, ws.total);
    }
    const bool bf16 = p->dtype == SAGE_BF16;
    const int dp = dp_of(p->d);
    const int nk_pad = (int)round_up(p->Nk, sage::kPad);
    sage::StatsArgs st{};
    st.x = p->v; st.sb = p->v_stride_b; st.sh = p->v_stride_h; st.sn = p->v_stride_n;
    st.cu = p->cu_seqlens_k; st.B = p->B; st.H = p->Hkv; st.N = p->Nk; st.d = p->d; st.dp = dp;
    st.chunks = ws.chunks; st.chunk_len = ws.chunk_len; st.want_minmax = fp8 ? 1 : 0;
    if (need_stats) {
        st.smooth = p->smooth_v ? 1 : 0;
        st.out_mean = p->smooth_v ? p->v_mean : nullptr;
        st.out_scale = fp8 ? p->v_scale : nullptr;
    }
    sage::QuantVArgs va{};
    va.v = p->v; va.sb = p->v_stride_b; va.sh = p->v_stride_h; va.sn = p->v_stride_n; va.cu = p->cu_seqlens_k;
    va.B = p->B; va.H = p->Hkv; va.N = p->Nk; va.npad = nk_pad; va.d = p->d; va.vt = p->vt;
    const bool vec = aligned(p->v, 16) && p->d % 8 == 0 && p->v_stride_b % 8 == 0 && p->v_stride_h % 8 == 0 &&
                     p->v_stride_n % 8 == 0;
    o.va = va;
    o.st = st;
    o.need_stats = need_stats;
    o.smooth = p->smooth_v != 0;
    o.bf16 = bf16;
    o.fp8 = fp8;
    o.vec = vec;
    o.wl = ws;
    o.ws_used = need_stats ? ws.total : 0;
    bind_v_ws(o, own_ws ? reinterpret_cast<uint8_t*>(p->workspace) : nullptr);
    return 0;
}

// Both parameter blocks of a fused call must describe the same K/V geometry.
int check_qkv_pair(const sage_quant_qk_params* qk, const sage_quant_v_params* v) {
    if (qk->dtype != v->dtype || qk->B != v->B || qk->Hkv != v->Hkv || qk->Nk != v->Nk || qk->d != v->d ||
        qk->cu_seqlens_k != v->cu_seqlens_k)
        return fail(SAGE_EINVAL, "K and V must share dtype, B, Hkv, Nk, head_dim and cu_seqlens_k");
    return SAGE_OK;
}
}  // namespace

int sage_quant_qk(const sage_quant_qk_params* p, void* stream) {
    QKPrep o;
    if (int r = prepare_qk(p, o)) return r;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (int r = hip_status(sage::launch_quant_qk(o.qa, o.ka, o.st, o.smooth, o.bf16, o.vec, s), "Q/K quantize launch"))
        return r;
    return ok();
}

int sage_quant_v(const sage_quant_v_params* p, void* stream) {
    VPrep o;
    if (int r = prepare_v(p, o)) return r;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (int r = hip_status(sage::launch_quant_v(o.va, o.st, o.need_stats, o.smooth, o.bf16, o.fp8, o.vec, s),
                           "V quantize launch"))
        return r;
    return ok();
}

int sage_quant_qkv(const sage_quant_qk_params* qk, const sage_quant_v_params* v, void* stream) {
    QKPrep a;
    VPrep b;
    if (int r = prepare_qk(qk, a)) return r;
    if (int r = prepare_v(v, b)) return r;
    if (int r = check_qkv_pair(qk, v)) return r;
    if (a.ws_used && b.ws_used) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.ws), b0 = reinterpret_cast<uintptr_t>(b.ws);
        if (a0 < b0 + b.ws_used && b0 < a0 + a.ws_used)
            return fail(SAGE_EINVAL, "the K and V workspaces overlap; the fused call needs one of each");
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (int r = hip_status(sage::launch_quant_qkv(a.qa, a.ka, a.st, a.smooth, b.va, b.st, b.need_stats, a.bf16, b.fp8,
                                                  a.vec && b.vec, s),
                           "Q/K/V quantize launch"))
        return r;
    return ok();
}

// ---------------------------------------------------------------------------
// The fused quantize call for callers that cannot allocate device memory.  Its
// statistics partials live in `scratch`, a file-scope device array that every
// GPU the library runs on holds for the life of the process.  In host code
// `scratch` names a host-side stand-in, not the device array: its device
// address comes from hipGetSymbolAddress, looked up once per device with that
// device current, and only that address is passed to kernels.
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;       // SAGE_QUANT_SCRATCH_BYTES in sage.h
static_assert(kScratchBytes == SAGE_QUANT_SCRATCH_BYTES, "scratch size and its public constant differ");
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_dev[kMaxDevices];                      // device address of `scratch`, per device
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
// Device address of `scratch` on the current device (looked up on the first
// call there).
int scratch_address(uint8_t** out) {
    int dev = -1;
    if (int r = hip_status(hipGetDevice(&dev), "hipGetDevice")) return r;
    if (dev < 0 || dev >= kMaxDevices) return fail(SAGE_EHIP, "device id %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        if (int r = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))
            return r;
        if (!ptr || !aligned(ptr, 256)) return fail(SAGE_EHIP, "scratch address %p unusable", ptr);
        g_scratch_dev[dev] = static_cast<uint8_t*>(ptr);
    }
    *out = g_scratch_dev[dev];
    return SAGE_OK;
}
}  // namespace

size_t sage_quant_qkv_noalloc_scratch_size(int B, int Hkv, int Nk, int d) {
    if (B < 1 || Hkv < 1 || Nk < 1 || d < 1 || d > 128) return 0;
    const size_t one = ws_layout(B, Hkv, Nk, d).total;  // a multiple of 256
    return 2 * one;
}

int sage_quant_qkv_noalloc(const sage_quant_qk_params* qk, const sage_quant_v_params* v, void* stream) {
    QKPrep a;
    VPrep b;
    if (int r = prepare_qk(qk, a, false)) return r;
    if (int r = prepare_v(v, b, false)) return r;
    if (int r = check_qkv_pair(qk, v)) return r;
    const size_t koff = 0, voff = a.ws_used;            // K partials, then V partials (256-byte multiples)
    const size_t need = a.ws_used + b.ws_used;
    if (need > kScratchBytes)
        return fail(SAGE_EINVAL,
                    "problem too large for the no-alloc call: its statistics need %zu bytes, the static scratch "
                    "holds %zu (use sage_quant_qkv with a workspace)",
                    need, kScratchBytes);
    uint8_t* base = nullptr;
    if (need) {
        if (int r = scratch_address(&base)) return r;
    }
    bind_qk_ws(a, base ? base + koff : nullptr);
    bind_v_ws(b, base ? base + voff : nullptr);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (int r = hip_status(sage::launch_quant_qkv(a.qa, a.ka, a.st, a.smooth, b.va, b.st, b.need_stats, a.bf16, b.fp8,
                                                  a.vec && b.vec, s),
                           "Q/K/V quantize launch (no-alloc)"))
        return r;
    return ok();
}

// Whether the attention kernel for these sizes quantizes Q itself: the
// 256-row tile kernel (FP8 V) at 128 padded channels, whole 8-channel slices,
// and quantization groups that never straddle two heads inside a tile of
// packed query heads.  (At 64 channels the key loop of a kernel that also
// quantizes Q compiles to slower code than the quantize pass saves.)
static bool q_fusable(int B, int Hq, int Hkv, int Nq, int d, int gran, int v_dtype, int is_causal, bool varlen) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || d < 1 || d > 128 || Hq % Hkv) return false;
    if (v_dtype != SAGE_V_FP8 || d <= 64 || d % 8 || !valid_gran(gran)) return false;
    const bool packed = !varlen && !is_causal && Hq > Hkv && Nq <= sage::kPackMaxNq;
    if (packed && Nq % (1 << q_group_shift(gran))) return false;
    return true;
}

int sage_attn_q_fusable(int B, int Hq, int Hkv, int Nq, int d, int gran, int v_dtype, int is_causal, int varlen) {
    return q_fusable(B, Hq, Hkv, Nq, d, gran, v_dtype, is_causal, varlen != 0) ? 1 : 0;
}

static int check_attn(const sage_attn_params* p, bool varlen) {
    if (int r = check_sizes(p->B, p->Hq, p->Hkv, p->Nq, p->Nk, p->d)) return r;
    if (!valid_gran(p->gran)) return fail(SAGE_EINVAL, "unknown qk_quant_gran %d", p->gran);
    if (p->v_dtype != SAGE_V_FP8 && p->v_dtype != SAGE_V_FP16) return fail(SAGE_EINVAL, "unknown v_dtype %d", p->v_dtype);
    if (p->pv_accum < SAGE_ACC_FP32 || p->pv_accum > SAGE_ACC_FP32_FP32)
        return fail(SAGE_EINVAL, "unknown pv_accum %d", p->pv_accum);
    if (!valid_dtype(p->in_dtype) || !valid_dtype(p->out_dtype)) return fail(SAGE_EINVAL, "unknown dtype");
    if ((!p->q && (!p->q8 || !p->q_scale)) || !p->k8 || !p->k_scale || !p->vt || !p->out)
        return fail(SAGE_EINVAL, "NULL tensor pointer");
    if (p->v_dtype == SAGE_V_FP8 && !p->v_scale) return fail(SAGE_EINVAL, "FP8 V needs v_scale");
    if (!aligned(p->q8, 16) || !aligned(p->k8, 16) || !aligned(p->vt, 16))
        return fail(SAGE_EINVAL, "q8/k8/vt must be 16-byte aligned");
    if (p->q) {
        if (!q_fusable(p->B, p->Hq, p->Hkv, p->Nq, p->d, p->gran, p->v_dtype, p->is_causal, varlen))
            return fail(SAGE_EUNSUPPORTED, "this call cannot take Q in its input precision (sage_attn_q_fusable)");
        if (!aligned(p->q, 16) || p->q_stride_n <= 0 || p->q_stride_h < 0 || (!varlen && p->q_stride_b < 0) ||
            p->q_stride_n % 8 || p->q_stride_h % 8 || (!varlen && p->q_stride_b % 8))
            return fail(SAGE_EINVAL, "q must be 16-byte aligned with non-negative strides that are multiples of 8");
    }
    if (!aligned(p->q_scale, 4) || !aligned(p->k_scale, 4) || (p->v_scale && !aligned(p->v_scale, 4)) ||
        (p->k_mean && !aligned(p->k_mean, 4)) || (p->v_mean && !aligned(p->v_mean, 4)) ||
        (p->lse && !aligned(p->lse, 4)))
        return fail(SAGE_EINVAL, "fp32 arrays must be 4-byte aligned");
    if (!aligned(p->out, 2)) return fail(SAGE_EINVAL, "out not 2-byte aligned");
    if (!std::isfinite(p->sm_scale)) return fail(SAGE_EINVAL, "sm_scale must be finite");
    if (p->o_stride_n <= 0 || p->o_stride_h < 0 || (!varlen && p->o_stride_b < 0))
        return fail(SAGE_EINVAL, "negative or zero output stride");
    return SAGE_OK;
}

static sage::AttnArgs attn_args(const sage_attn_params* p) {
    sage::AttnArgs a{};
    a.q8 = p->q8; a.qs = p->q_scale; a.k8 = p->k8; a.ks = p->k_scale; a.kmean = p->k_mean;
    a.qraw = p->q; a.qsb = p->q_stride_b; a.qsh = p->q_stride_h; a.qsn = p->q_stride_n;
    a.q_bf16 = p->in_dtype == SAGE_BF16 ? 1 : 0;
    a.vt = p->vt; a.vs = p->v_scale; a.vmean = p->v_mean; a.out = p->out; a.lse = p->lse;
    a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nq = p->Nq; a.Nk = p->Nk; a.d = p->d;
    a.nq_pad = (int)round_up(p->Nq, sage::kPad);
    a.nk_pad = (int)round_up(p->Nk, sage::kPad);
    a.gq_shift = q_group_shift(p->gran);
    a.gk_shift = k_group_shift(p->gran);
    a.causal = p->is_causal ? 1 : 0;
    a.sm_scale = p->sm_scale > 0.f ? p->sm_scale : (float)(1.0 / std::sqrt((double)p->d));
    a.ob = p->o_stride_b; a.oh = p->o_stride_h; a.on = p->o_stride_n;
    a.out_vec4 = aligned(p->out, 8) && p->o_stride_n % 4 == 0 && p->o_stride_h % 4 == 0 && p->o_stride_b % 4 == 0;
    a.out_vec8 = aligned(p->out, 16) && p->o_stride_n % 8 == 0 && p->o_stride_h % 8 == 0 && p->o_stride_b % 8 == 0 &&
                 p->d % 8 == 0;
    a.n_qtiles = (int)((p->Nq + sage::kBQ - 1) / sage::kBQ);
    a.num_wg = p->B * p->Hq * a.n_qtiles;
    return a;
}

// Few queries per head with grouped K/V heads: one workgroup takes the rows
// of every query head that shares a K/V head (FP8 V, non-causal, dense).
static int pack_gqa(const sage_attn_params* p) {
    return p->v_dtype == SAGE_V_FP8 && !p->is_causal && p->Hq > p->Hkv && p->Nq <= sage::kPackMaxNq;
}

static int pv_kind(const sage_attn_params* p) {
    return p->v_dtype == SAGE_V_FP8 ? 0 : (p->in_dtype == SAGE_BF16 ? 2 : 1);
}

int sage_attn_fwd(const sage_attn_params* p, void* stream) {
    if (!p) return fail(SAGE_EINVAL, "params is NULL");
    if (p->struct_size < sizeof(sage_attn_params)) return fail(SAGE_EINVAL, "struct_size too small");
    if (int r = check_attn(p, false)) return r;
    sage::AttnArgs a = attn_args(p);
    a.pack_gqa = pack_gqa(p);
    if (int r = hip_status(sage::launch_attn(a, dp_of(p->d), pv_kind(p), p->out_dtype == SAGE_BF16,
                                             reinterpret_cast<hipStream_t>(stream)),
                           "attention launch"))
        return r;
    return ok();
}

int sage_attn_varlen_fwd(const sage_attn_varlen_params* p, void* stream) {
    if (!p) return fail(SAGE_EINVAL, "params is NULL");
    if (p->base.struct_size < sizeof(sage_attn_varlen_params))
        return fail(SAGE_EINVAL, "struct_size too small (pass sizeof(sage_attn_varlen_params))");
    if (int r = check_attn(&p->base, true)) return r;
    if (!p->cu_seqlens_q || !p->cu_seqlens_k) return fail(SAGE_EINVAL, "varlen needs cu_seqlens_q and cu_seqlens_k");
    if (!aligned(p->cu_seqlens_q, 4) || !aligned(p->cu_seqlens_k, 4)) return fail(SAGE_EINVAL, "cu_seqlens misaligned");
    if (p->base.lse && p->total_q < 1) return fail(SAGE_EINVAL, "total_q must be >= 1 with lse");
    sage::AttnArgs a = attn_args(&p->base);
    a.cu_q = p->cu_seqlens_q;
    a.cu_k = p->cu_seqlens_k;
    a.lse_varlen = 1;
    a.total_q = p->total_q;
    a.out_vec4 = aligned(p->base.out, 8) && p->base.o_stride_n % 4 == 0 && p->base.o_stride_h % 4 == 0;
    a.out_vec8 = aligned(p->base.out, 16) && p->base.o_stride_n % 8 == 0 && p->base.o_stride_h % 8 == 0 &&
                 p->base.d % 8 == 0;
    if (int r = hip_status(sage::launch_attn(a, dp_of(p->base.d), pv_kind(&p->base), p->base.out_dtype == SAGE_BF16,
                                             reinterpret_cast<hipStream_t>(stream)),
                           "varlen attention launch"))
        return r;
    return ok();
}

int sage_debug_qk_scores(const sage_attn_params* p, int mode, void* scores, void* stream) {
    if (!p) return fail(SAGE_EINVAL, "params is NULL");
    if (p->struct_size < sizeof(sage_attn_params)) return fail(SAGE_EINVAL, "struct_size too small");
    if (int r = check_sizes(p->B, p->Hq, p->Hkv, p->Nq, p->Nk, p->d)) return r;
    if (mode != 0 && mode != 1) return fail(SAGE_EINVAL, "mode must be 0 or 1");
    if (!p->q8 || !p->k8 || !scores) return fail(SAGE_EINVAL, "NULL pointer");
    if (!aligned(p->q8, 16) || !aligned(p->k8, 16) || !aligned(scores, 8))
        return fail(SAGE_EINVAL, "misaligned pointer");
    sage::AttnArgs a = attn_args(p);
    a.dbg = scores;
    a.dbg_mode = mode;
    if (int r = hip_status(sage::launch_qk_scores(a, dp_of(p->d), reinterpret_cast<hipStream_t>(stream)),
                           "score dump launch"))
        return r;
    return ok();
}

int sage_debug_qk_scores_varlen(const sage_attn_varlen_params* p, void* checksums, void* stream) {
    if (!p) return fail(SAGE_EINVAL, "params is NULL");
    if (p->base.struct_size < sizeof(sage_attn_varlen_params))
        return fail(SAGE_EINVAL, "struct_size too small (pass sizeof(sage_attn_varlen_params))");
    const sage_attn_params* b = &p->base;
    if (int r = check_sizes(b->B, b->Hq, b->Hkv, b->Nq, b->Nk, b->d)) return r;
    if (!b->q8 || !b->k8 || !checksums || !p->cu_seqlens_q || !p->cu_seqlens_k)
        return fail(SAGE_EINVAL, "NULL pointer");
    if (!aligned(b->q8, 16) || !aligned(b->k8, 16) || !aligned(checksums, 8) || !aligned(p->cu_seqlens_q, 4) ||
        !aligned(p->cu_seqlens_k, 4))
        return fail(SAGE_EINVAL, "misaligned pointer");
    if (p->total_q < 1) return fail(SAGE_EINVAL, "total_q must be >= 1");
    sage::AttnArgs a = attn_args(b);
    a.cu_q = p->cu_seqlens_q;
    a.cu_k = p->cu_seqlens_k;
    a.total_q = p->total_q;
    a.dbg = checksums;
    a.dbg_mode = 1;
    if (int r = hip_status(sage::launch_qk_scores(a, dp_of(b->d), reinterpret_cast<hipStream_t>(stream)),
                           "varlen score checksum launch"))
        return r;
    return ok();
}

namespace {
struct SplitPlan {
    int splits, split_len;
    size_t parts_bytes, lse_bytes, total;
};
// Key ranges of n_splits requested splits: multiples of 128 keys, none empty.
SplitPlan split_plan(int B, int Hq, int Nq, int Nk, int d, int n_splits) {
    SplitPlan s{};
    const int64_t per = (Nk + (int64_t)n_splits - 1) / n_splits;
    s.split_len = (int)round_up(per, sage::kPad);
    s.splits = (int)((Nk + (int64_t)s.split_len - 1) / s.split_len);
    const size_t rows = (size_t)s.splits * B * Hq * Nq;
    s.parts_bytes = (rows * d * 4 + 255) / 256 * 256;     // fp32 partial outputs
    s.lse_bytes = (rows * 4 + 255) / 256 * 256;
    s.total = s.parts_bytes + s.lse_bytes;
    return s;
}
}  // namespace

size_t sage_attn_splitkv_workspace_size(int B, int Hq, int Nq, int Nk, int d, int n_splits) {
    if (B < 1 || Hq < 1 || Nq < 1 || Nk < 1 || d < 1 || d > 128 || n_splits < 1 || n_splits > 64) return 0;
    return split_plan(B, Hq, Nq, Nk, d, n_splits).total;
}

int sage_attn_fwd_splitkv(const sage_attn_params* p, int n_splits, void* workspace, size_t workspace_bytes,
                          void* stream) {
    if (!p) return fail(SAGE_EINVAL, "params is NULL");
    if (p->struct_size < sizeof(sage_attn_params)) return fail(SAGE_EINVAL, "struct_size too small");
    if (int r = check_attn(p, false)) return r;
    if (n_splits < 1 || n_splits > 64) return fail(SAGE_EINVAL, "n_splits %d must be 1..64", n_splits);
    if (p->is_causal) return fail(SAGE_EUNSUPPORTED, "split-KV is non-causal only");
    const SplitPlan sp = split_plan(p->B, p->Hq, p->Nq, p->Nk, p->d, n_splits);
    if (!workspace || !aligned(workspace, 256)) return fail(SAGE_EINVAL, "workspace NULL or not 256-byte aligned");
    if (workspace_bytes < sp.total)
        return fail(SAGE_EINVAL, "workspace too small: %zu < %zu bytes", workspace_bytes, sp.total);
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const int64_t d = p->d, rows = (int64_t)p->B * p->Hq * p->Nq;
    // partial results of split s: fp32 out [B][Hq][Nq][d] and LSE [B][Hq][Nq]
    sage::AttnArgs a = attn_args(p);
    a.out = ws;
    a.out_f32 = 1;
    a.out_vec8 = 0;                                     // (fp32 partial results: the 8-byte path)
    a.ob = (int64_t)p->Hq * p->Nq * d;
    a.oh = (int64_t)p->Nq * d;
    a.on = d;
    a.out_vec4 = d % 4 == 0;
    a.lse = reinterpret_cast<float*>(ws + sp.parts_bytes);
    a.n_splits = sp.splits;
    a.split_len = sp.split_len;
    a.split_out = rows * d;
    a.split_lse = rows;
    a.pack_gqa = pack_gqa(p);
    const bool out_bf16 = p->out_dtype == SAGE_BF16;
    if (int r = hip_status(sage::launch_attn(a, dp_of(p->d), pv_kind(p), out_bf16, st), "split-KV attention launch"))
        return r;
    sage::MergeArgs m{};
    m.parts = ws;
    m.parts_f32 = 1;
    m.ps = rows * d;
    m.pb = a.ob;
    m.ph = a.oh;
    m.pn = d;
    m.lse_parts = a.lse;
    m.out = p->out;
    m.ob = p->o_stride_b;
    m.oh = p->o_stride_h;
    m.on = p->o_stride_n;
    m.lse = p->lse;
    m.S = sp.splits;
    m.B = p->B;
    m.H = p->Hq;
    m.N = p->Nq;
    m.d = p->d;
    const bool vec = p->d % 8 == 0 && aligned(p->out, 16) && p->o_stride_b % 8 == 0 && p->o_stride_h % 8 == 0 &&
                     p->o_stride_n % 8 == 0;
    if (int r = hip_status(sage::launch_merge(m, out_bf16, vec, st), "split-KV merge launch")) return r;
    return ok();
}

int sage_merge_states(const sage_merge_params* p, void* stream) {
    if (!p) return fail(SAGE_EINVAL, "params is NULL");
    if (p->struct_size < sizeof(sage_merge_params)) return fail(SAGE_EINVAL, "struct_size too small");
    if (p->n_parts < 1 || p->n_parts > 64) return fail(SAGE_EINVAL, "n_parts %d must be 1..64", p->n_parts);
    if (p->B < 1 || p->H < 1 || p->N < 1) return fail(SAGE_EINVAL, "sizes must be >= 1 (B=%d H=%d N=%d)", p->B, p->H, p->N);
    if (p->d < 1 || p->d > 1024) return fail(SAGE_EINVAL, "d %d must be 1..1024", p->d);
    if ((int64_t)p->B * p->H * p->N > ((int64_t)1 << 40) / p->d) return fail(SAGE_EINVAL, "sizes too large");
    if (!valid_dtype(p->dtype)) return fail(SAGE_EINVAL, "invalid dtype %d", p->dtype);
    if (!p->parts || !p->lse_parts || !p->out) return fail(SAGE_EINVAL, "NULL pointer");
    if (!aligned(p->parts, 2) || !aligned(p->out, 2) || !aligned(p->lse_parts, 4) || (p->lse && !aligned(p->lse, 4)))
        return fail(SAGE_EINVAL, "misaligned pointer");
    sage::MergeArgs a{};
    a.parts = p->parts;
    a.ps = p->ps_s;
    a.pb = p->ps_b;
    a.ph = p->ps_h;
    a.pn = p->ps_n;
    a.lse_parts = p->lse_parts;
    a.out = p->out;
    a.ob = p->o_stride_b;
    a.oh = p->o_stride_h;
    a.on = p->o_stride_n;
    a.lse = p->lse;
    a.S = p->n_parts;
    a.B = p->B;
    a.H = p->H;
    a.N = p->N;
    a.d = p->d;
    // 16-byte pieces of every row: d and every stride a multiple of 8 elements, bases 16-byte aligned
    const bool vec = p->d % 8 == 0 && aligned(p->parts, 16) && aligned(p->out, 16) && p->ps_s % 8 == 0 &&
                     p->ps_b % 8 == 0 && p->ps_h % 8 == 0 && p->ps_n % 8 == 0 && p->o_stride_b % 8 == 0 &&
                     p->o_stride_h % 8 == 0 && p->o_stride_n % 8 == 0;
    if (int r = hip_status(sage::launch_merge(a, p->dtype == SAGE_BF16, vec, reinterpret_cast<hipStream_t>(stream)),
                           "merge launch"))
        return r;
    return ok();
}

}  // extern "C"
