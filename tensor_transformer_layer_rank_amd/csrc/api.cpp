// C-ABI front end of libtpshard: host-side validation, workspace carving and dispatch
// to the gfx950 kernels. Every check runs before the first HIP call, so a rejected call
// launches nothing. The public contract is documented in include/tpshard.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tp_internal.h"

namespace {

thread_local std::string g_last_error;

tp_status fail(tp_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

tp_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return TP_OK;
    return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr size_t WS_ALIGN = 256;
constexpr int64_t SKINNY_MAX_T = 64;   // rows at or below which the decode (weight-streaming) kernels run
// The MFMA GEMM tiles address a 256-row activation block with 32-bit element offsets
// (row * lda + column): a contraction length / activation leading dimension must stay below
// 2^31 / 256 = 2^23 elements.
constexpr int64_t LD_LIMIT = (int64_t)1 << 23;

tp_status check_ld(const char* fn, const char* what, int64_t v) {
    if (v >= LD_LIMIT)
        return fail(TP_ERR_UNSUPPORTED, "%s: %s = %lld (the 16-bit and fp8 paths offer fewer than 2^23)", fn, what,
                    (long long)v);
    return TP_OK;
}

// carve consecutive 256-byte aligned sub-buffers out of a workspace
struct Carver {
    unsigned char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<unsigned char*>(b)) {}
    void* take(size_t bytes) {
        void* p = base ? base + off : nullptr;
        off += round_up(bytes, WS_ALIGN);
        return p;
    }
};

// ---- kernel timing ------------------------------------------------------------------------
struct ProfRec {
    std::string name;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<hipEvent_t> g_pool;
size_t g_pool_used = 0;
std::vector<ProfRec> g_recs;
thread_local bool t_pending = false;
thread_local std::string t_pending_name;
thread_local hipEvent_t t_pending_start;
constexpr size_t PROF_MAX = 65536;

hipEvent_t pool_event() {
    if (g_pool_used == g_pool.size()) {
        hipEvent_t e;
        // timing only: no system-scope cache write-back and invalidate when the event is
        // recorded (that fence costs microseconds and slows the kernels that follow)
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
        g_pool.push_back(e);
    }
    return g_pool[g_pool_used++];
}

}  // namespace

namespace tpk {

void prof_begin(const char* name, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    t_pending = false;
    if (!g_prof_on || g_recs.size() >= PROF_MAX) return;
    hipEvent_t a = pool_event();
    if (!a) return;
    if (hipEventRecord(a, s) != hipSuccess) return;
    t_pending = true;
    t_pending_name = name;
    t_pending_start = a;
}

void prof_end(hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!t_pending) return;
    t_pending = false;
    hipEvent_t b = pool_event();
    if (!b) return;
    if (hipEventRecord(b, s) != hipSuccess) return;
    g_recs.push_back(ProfRec{t_pending_name, t_pending_start, b});
}

}  // namespace tpk

extern "C" {

int tp_abi_version(void) { return TP_ABI_VERSION; }

const char* tp_status_string(tp_status st) {
    switch (st) {
        case TP_OK: return "TP_OK";
        case TP_ERR_NULL_POINTER: return "TP_ERR_NULL_POINTER";
        case TP_ERR_BAD_SHAPE: return "TP_ERR_BAD_SHAPE";
        case TP_ERR_BAD_DTYPE: return "TP_ERR_BAD_DTYPE";
        case TP_ERR_MISALIGNED: return "TP_ERR_MISALIGNED";
        case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE";
        case TP_ERR_UNSUPPORTED: return "TP_ERR_UNSUPPORTED";
        case TP_ERR_HIP: return "TP_ERR_HIP";
    }
    return "TP_ERR_UNKNOWN";
}

const char* tp_last_error(void) { return g_last_error.c_str(); }

tp_status tp_profile_enable(int on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = on != 0;
    return TP_OK;
}

tp_status tp_profile_reset(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_recs.clear();
    g_pool_used = 0;
    return TP_OK;
}

tp_status tp_mfma_rate_probe(const void* operands, float* out, int64_t n_workgroups, int64_t iters, void* stream) {
    const char* fn = "tp_mfma_rate_probe";
    if (!operands || !out) return fail(TP_ERR_NULL_POINTER, "%s: operands and out must be non-NULL", fn);
    if (!aligned(operands, 16) || !aligned(out, 4)) return fail(TP_ERR_MISALIGNED, "%s: operands 16-byte, out 4-byte aligned", fn);
    if (n_workgroups < 1 || n_workgroups > (1 << 20) || iters < 1 || iters > ((int64_t)1 << 30))
        return fail(TP_ERR_BAD_SHAPE, "%s: need 1 <= n_workgroups <= 2^20 and 1 <= iters <= 2^30", fn);
    return from_hip(tpk::mfma_rate(operands, out, n_workgroups, iters, as_stream(stream)), fn);
}

tp_status tp_hbm_read_probe(const void* buf, int64_t bytes_per_workgroup, int64_t n_workgroups, unsigned* out,
                            void* stream) {
    const char* fn = "tp_hbm_read_probe";
    if (!buf || !out) return fail(TP_ERR_NULL_POINTER, "%s: buf and out must be non-NULL", fn);
    if (!aligned(buf, 16) || !aligned(out, 4)) return fail(TP_ERR_MISALIGNED, "%s: buf 16-byte, out 4-byte aligned", fn);
    if (n_workgroups < 1 || n_workgroups > (1 << 20) || bytes_per_workgroup < 8192 ||
        bytes_per_workgroup > ((int64_t)1 << 34) || bytes_per_workgroup % 8192)
        return fail(TP_ERR_BAD_SHAPE, "%s: need 1 <= n_workgroups <= 2^20 and bytes_per_workgroup a multiple of 8192 "
                    "in [8192, 2^34]", fn);
    return from_hip(tpk::hbm_read(buf, bytes_per_workgroup, n_workgroups, out, as_stream(stream)), fn);
}

tp_status tp_profile_read(const char* prefix, double* total_ms, int64_t* launches) {
    if (!prefix || !total_ms || !launches) return fail(TP_ERR_NULL_POINTER, "tp_profile_read: NULL argument");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    double tot = 0.0;
    int64_t n = 0;
    const size_t plen = strlen(prefix);
    for (const ProfRec& r : g_recs) {
        if (r.name.compare(0, plen, prefix) != 0) continue;
        hipError_t e = hipEventSynchronize(r.b);
        if (e != hipSuccess) return from_hip(e, "tp_profile_read");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess) return from_hip(e, "tp_profile_read");
        tot += ms;
        ++n;
    }
    *total_ms = tot;
    *launches = n;
    return TP_OK;
}

// ---- linear layers ----------------------------------------------------------------------

size_t tp_linear_workspace_size(int64_t T, int64_t K, int64_t N, tp_dtype in_dt) {
    if (T <= 0 || K <= 0 || N <= 0) return 0;
    if (in_dt == TP_FP8_E4M3) return round_up(tpk::gemm_f8_split_bytes(T, N, K, 0), WS_ALIGN);
    if (in_dt != TP_BF16 && in_dt != TP_F16) return 0;
    if (T > SKINNY_MAX_T) return round_up(tpk::gemm_bf16_split_bytes(T, N, K, 0), WS_ALIGN);
    return round_up(tpk::skinny_partials_bytes(T, N, K), WS_ALIGN);
}

static tp_status check_ws(const char* fn, const void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return TP_OK;
    if (!ws || ws_bytes < need)
        return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);
    if (!aligned(ws, 16)) return fail(TP_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", fn);
    return TP_OK;
}

static tp_status check_f8(const char* fn, const void* X, const void* W, const void* Y,
                          int64_t K, int64_t N, const tp_fp8_scales* q) {
    if (!q) return fail(TP_ERR_NULL_POINTER, "%s: fp8 operands need their scales (q is NULL)", fn);
    if (!(q->x_scale > 0.0f) || !(q->w_scale > 0.0f))
        return fail(TP_ERR_BAD_SHAPE, "%s: fp8 scales must be positive (x %g, w %g)", fn, (double)q->x_scale,
                    (double)q->w_scale);
    if (!aligned(X, 16) || !aligned(W, 16) || !aligned(Y, 16))
        return fail(TP_ERR_MISALIGNED, "%s: fp8 path needs 16-byte aligned X, W and Y", fn);
    if (K % 16 || N % 16)
        return fail(TP_ERR_MISALIGNED, "%s: fp8 path needs K and N multiples of 16 (K=%lld N=%lld)", fn,
                    (long long)K, (long long)N);
    return TP_OK;
}

static tp_status check_bf16_gemm(const char* fn, const void* X, const void* W, const void* Y,
                                 int64_t K, int64_t N, int64_t ldy) {
    if (!aligned(X, 16) || !aligned(W, 16) || !aligned(Y, 16))
        return fail(TP_ERR_MISALIGNED, "%s: bf16 path needs 16-byte aligned X, W and Y", fn);
    if (K % 8 || N % 8 || ldy % 8)
        return fail(TP_ERR_MISALIGNED, "%s: bf16 path needs K, N and ldy multiples of 8 (K=%lld N=%lld ldy=%lld)",
                    fn, (long long)K, (long long)N, (long long)ldy);
    return TP_OK;
}

// tp_column_linear in two halves: the argument checks (pure host code) choose the kernel path
// and the workspace it needs; the launch runs it. The allocation-free variant shares both.
struct ColumnPlan {
    enum { F32, FP8, SKINNY, MFMA16 } path;
    int kind;       // store kind of the prefill tiles (0 bf16, 1 fp16, 2 fp32)
    int rk;         // epilogue of the few-row reduce (0 fp32, 2 bf16, 3 bf16 ReLU, 5 fp16, 6 fp16 ReLU, 7 fp32 ReLU)
    int f16;        // fp16 operands (else bf16)
    size_t need;    // tp_linear_workspace_size of the call
};

static tp_status column_linear_check(const char* fn, const void* X, const void* W_shard, void* Y, int64_t T,
                                     int64_t K, int64_t N, int64_t ldy, tp_dtype in_dt, tp_dtype out_dt, tp_act act,
                                     const tp_fp8_scales* q, ColumnPlan* p) {
    if (!X || !W_shard || !Y) return fail(TP_ERR_NULL_POINTER, "%s: X, W_shard and Y must be non-NULL", fn);
    if (T <= 0 || K <= 0 || N <= 0)
        return fail(TP_ERR_BAD_SHAPE, "%s: sizes must be positive (T=%lld K=%lld N=%lld)", fn, (long long)T,
                    (long long)K, (long long)N);
    if (ldy < N) return fail(TP_ERR_BAD_SHAPE, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
    if (act != TP_ACT_NONE && act != TP_ACT_RELU) return fail(TP_ERR_BAD_SHAPE, "%s: unknown activation %d", fn, (int)act);
    *p = ColumnPlan{ColumnPlan::F32, 0, 0, 0, 0};
    if (in_dt == TP_F32) {
        if (out_dt != TP_F32) return fail(TP_ERR_BAD_DTYPE, "%s: fp32 input needs fp32 output", fn);
        if (!aligned(X, 4) || !aligned(W_shard, 4) || !aligned(Y, 4))
            return fail(TP_ERR_MISALIGNED, "%s: fp32 pointers must be 4-byte aligned", fn);
        return TP_OK;
    }
    p->kind = out_dt == TP_BF16 ? 0 : (out_dt == TP_F16 ? 1 : 2);
    if (in_dt == TP_FP8_E4M3) {
        if (out_dt != TP_BF16 && out_dt != TP_F16 && out_dt != TP_F32)
            return fail(TP_ERR_BAD_DTYPE, "%s: fp8 input needs bf16, fp16 or fp32 output", fn);
        tp_status st = check_f8(fn, X, W_shard, Y, K, N, q);
        if (st != TP_OK) return st;
        if (ldy % 8) return fail(TP_ERR_MISALIGNED, "%s: ldy must be a multiple of 8", fn);
        st = check_ld(fn, "K", K);
        if (st != TP_OK) return st;
        p->path = ColumnPlan::FP8;
        p->need = tp_linear_workspace_size(T, K, N, in_dt);
        return TP_OK;
    }
    if (in_dt != TP_BF16 && in_dt != TP_F16) return fail(TP_ERR_BAD_DTYPE, "%s: input dtype %d not offered", fn, (int)in_dt);
    if (out_dt != TP_BF16 && out_dt != TP_F16 && out_dt != TP_F32)
        return fail(TP_ERR_BAD_DTYPE, "%s: bf16/fp16 input needs bf16, fp16 or fp32 output", fn);
    tp_status st = check_bf16_gemm(fn, X, W_shard, Y, K, N, ldy);
    if (st != TP_OK) return st;
    st = check_ld(fn, "K", K);
    if (st != TP_OK) return st;
    p->f16 = in_dt == TP_F16;
    p->need = tp_linear_workspace_size(T, K, N, in_dt);
    if (T <= SKINNY_MAX_T) {
        const bool relu = act == TP_ACT_RELU;
        p->rk = out_dt == TP_F32 ? (relu ? 7 : 0) : out_dt == TP_BF16 ? (relu ? 3 : 2) : (relu ? 6 : 5);
        p->path = ColumnPlan::SKINNY;
        return TP_OK;
    }
    p->path = ColumnPlan::MFMA16;
    return TP_OK;
}

// ws may be smaller than p.need on the prefill paths only (their tiles then all run whole)
static hipError_t column_linear_launch(const ColumnPlan& p, const void* X, const void* W_shard, void* Y, int64_t T,
                                       int64_t K, int64_t N, int64_t ldy, tp_act act, const tp_fp8_scales* q,
                                       void* ws, size_t ws_bytes, hipStream_t s) {
    const int relu = act == TP_ACT_RELU;
    switch (p.path) {
        case ColumnPlan::F32:
            return tpk::gemm_f32(static_cast<const float*>(X), static_cast<const float*>(W_shard),
                                 static_cast<float*>(Y), T, N, K, K, N, ldy, relu, 0, s);
        case ColumnPlan::FP8:
            return tpk::gemm_f8_store(X, W_shard, Y, T, N, K, K, N, ldy, p.kind, relu, q->x_scale * q->w_scale, 1.0f,
                                      ws, ws_bytes, s);
        case ColumnPlan::SKINNY:
            return tpk::skinny_linear(X, W_shard, static_cast<float*>(ws), T, N, K, K, Y, ldy, p.rk, s, p.f16);
        case ColumnPlan::MFMA16:
            return (p.f16 ? tpk::gemm_f16_store : tpk::gemm_bf16_store)(X, W_shard, Y, T, N, K, K, N, ldy, p.kind,
                                                                        relu, ws, ws_bytes, s);
    }
    return hipErrorInvalidValue;
}

tp_status tp_column_linear(const void* X, const void* W_shard, void* Y, int64_t T, int64_t K,
                           int64_t N, int64_t ldy, tp_dtype in_dt, tp_dtype out_dt, tp_act act,
                           const tp_fp8_scales* q, void* workspace, size_t ws_bytes,
                           void* stream) {
    const char* fn = "tp_column_linear";
    ColumnPlan p;
    tp_status st = column_linear_check(fn, X, W_shard, Y, T, K, N, ldy, in_dt, out_dt, act, q, &p);
    if (st != TP_OK) return st;
    st = check_ws(fn, workspace, ws_bytes, p.need);
    if (st != TP_OK) return st;
    return from_hip(column_linear_launch(p, X, W_shard, Y, T, K, N, ldy, act, q, workspace, ws_bytes, as_stream(stream)),
                    fn);
}

tp_status tp_column_linear_noalloc(const void* X, const void* W_shard, void* Y, int64_t T, int64_t K, int64_t N,
                                   int64_t ldy, tp_dtype in_dt, tp_dtype out_dt, tp_act act, const tp_fp8_scales* q,
                                   void* stream) {
    const char* fn = "tp_column_linear_noalloc";
    ColumnPlan p;
    tp_status st = column_linear_check(fn, X, W_shard, Y, T, K, N, ldy, in_dt, out_dt, act, q, &p);
    if (st != TP_OK) return st;
    if (p.path == ColumnPlan::SKINNY && p.need > (size_t)TP_NOALLOC_SCRATCH_BYTES)
        return fail(TP_ERR_UNSUPPORTED, "%s: T=%lld K=%lld N=%lld needs %zu bytes of partial sums; the library's "
                    "scratch holds %zu", fn, (long long)T, (long long)K, (long long)N, p.need,
                    (size_t)TP_NOALLOC_SCRATCH_BYTES);
    hipStream_t s = as_stream(stream);
    void* scratch = nullptr;
    if (p.path != ColumnPlan::F32) {
        hipError_t e = tpk::noalloc_scratch(s, &scratch);
        if (e != hipSuccess) return from_hip(e, fn);
    }
    return from_hip(column_linear_launch(p, X, W_shard, Y, T, K, N, ldy, act, q, scratch,
                                         scratch ? (size_t)TP_NOALLOC_SCRATCH_BYTES : 0, s),
                    fn);
}

tp_status tp_row_linear_partial(const void* X_shard, const void* W_shard, float* Y_partial,
                                int64_t T, int64_t K_shard, int64_t N, tp_dtype in_dt,
                                int accumulate, const tp_fp8_scales* q, void* workspace,
                                size_t ws_bytes, void* stream) {
    (void)q;
    if (!X_shard || !W_shard || !Y_partial)
        return fail(TP_ERR_NULL_POINTER, "tp_row_linear_partial: X_shard, W_shard and Y_partial must be non-NULL");
    if (T <= 0 || K_shard <= 0 || N <= 0)
        return fail(TP_ERR_BAD_SHAPE, "tp_row_linear_partial: sizes must be positive (T=%lld K=%lld N=%lld)",
                    (long long)T, (long long)K_shard, (long long)N);
    hipStream_t s = as_stream(stream);
    if (in_dt == TP_F32) {
        if (!aligned(X_shard, 4) || !aligned(W_shard, 4) || !aligned(Y_partial, 4))
            return fail(TP_ERR_MISALIGNED, "tp_row_linear_partial: fp32 pointers must be 4-byte aligned");
        return from_hip(tpk::gemm_f32(static_cast<const float*>(X_shard), static_cast<const float*>(W_shard),
                                      Y_partial, T, N, K_shard, K_shard, N, N, 0, accumulate != 0, s),
                        "tp_row_linear_partial");
    }
    if (in_dt == TP_FP8_E4M3) {
        tp_status st = check_f8("tp_row_linear_partial", X_shard, W_shard, Y_partial, K_shard, N, q);
        if (st != TP_OK) return st;
        st = check_ld("tp_row_linear_partial", "K_shard", K_shard);
        if (st != TP_OK) return st;
        st = check_ws("tp_row_linear_partial", workspace, ws_bytes, tp_linear_workspace_size(T, K_shard, N, in_dt));
        if (st != TP_OK) return st;
        return from_hip(tpk::gemm_f8_store(X_shard, W_shard, Y_partial, T, N, K_shard, K_shard, N, N,
                                           accumulate ? 3 : 2, 0, q->x_scale * q->w_scale, 1.0f, workspace,
                                           ws_bytes, s),
                        "tp_row_linear_partial");
    }
    if (in_dt != TP_BF16 && in_dt != TP_F16)
        return fail(TP_ERR_BAD_DTYPE, "tp_row_linear_partial: input dtype %d not offered", (int)in_dt);
    tp_status st = check_bf16_gemm("tp_row_linear_partial", X_shard, W_shard, Y_partial, K_shard, N, N);
    if (st != TP_OK) return st;
    st = check_ld("tp_row_linear_partial", "K_shard", K_shard);
    if (st != TP_OK) return st;
    const int f16 = in_dt == TP_F16;
    st = check_ws("tp_row_linear_partial", workspace, ws_bytes, tp_linear_workspace_size(T, K_shard, N, in_dt));
    if (st != TP_OK) return st;
    if (T <= SKINNY_MAX_T) {
        return from_hip(tpk::skinny_linear(X_shard, W_shard, static_cast<float*>(workspace), T, N, K_shard, K_shard,
                                           Y_partial, N, accumulate ? 1 : 0, s, f16),
                        "tp_row_linear_partial");
    }
    return from_hip((f16 ? tpk::gemm_f16_store : tpk::gemm_bf16_store)(X_shard, W_shard, Y_partial, T, N, K_shard,
                                                                       K_shard, N, N, accumulate ? 3 : 2, 0,
                                                                       workspace, ws_bytes, s),
                    "tp_row_linear_partial");
}

// ---- MLP shard ------------------------------------------------------------------------------

size_t tp_mlp_workspace_size(int64_t T, int64_t H, int64_t I_shard, tp_mlp_kind kind,
                             tp_dtype in_dt, tp_dtype h_dt) {
    (void)kind;
    if (T <= 0 || H <= 0 || I_shard <= 0) return 0;
    if (in_dt == TP_F32) return round_up((size_t)(T * I_shard) * 4, WS_ALIGN);
    if (in_dt == TP_F16 && h_dt != TP_F16) return 0;                 // fp16 operands keep h in fp16
    if (in_dt != TP_BF16 && in_dt != TP_F16) return 0;
    if (h_dt != TP_BF16 && h_dt != TP_F16) return 0;
    if (in_dt == TP_BF16 && h_dt == TP_F16 && T <= SKINNY_MAX_T) return 0;
    size_t bytes = round_up((size_t)(T * I_shard) * 2, WS_ALIGN);   // h
    if (in_dt == TP_BF16 && h_dt == TP_F16) bytes += round_up((size_t)(I_shard * H) * 2, WS_ALIGN);   // W_down in fp16
    if (T <= SKINNY_MAX_T) {
        const size_t first = kind == TP_MLP_SWIGLU ? tpk::skinny_swiglu_partials_bytes(T, I_shard, H)
                                                   : tpk::skinny_partials_bytes(T, I_shard, H);
        const size_t second = tpk::skinny_partials_bytes(T, H, I_shard);
        bytes += round_up(first > second ? first : second, WS_ALIGN);
    } else {
        const size_t first = tpk::gemm_bf16_split_bytes(T, I_shard, H, kind == TP_MLP_SWIGLU ? 1 : 0);
        const size_t second = tpk::gemm_bf16_split_bytes(T, H, I_shard, 0);
        bytes += round_up(first > second ? first : second, WS_ALIGN);
    }
    return bytes;
}

// The bf16 MLP shard on T rows (validated arguments): gate/up (SwiGLU, or ReLU without W_up)
// into h in the workspace, then the down projection's fp32 partial. `need` is
// tp_mlp_workspace_size of the same arguments. h_f16 (T > 64 only): h is stored in fp16, W_down
// is converted to fp16 into the workspace, and the down projection runs on fp16 operands.
// in_f16: every operand is fp16 already, and so is h (no conversion).
static hipError_t mlp_bf16(const void* X, const void* W_gate, const void* W_up, const void* W_down, float* Y,
                           int64_t T, int64_t H, int64_t I, tp_mlp_kind kind, void* workspace, size_t need,
                           hipStream_t s, bool h_f16 = false, bool in_f16 = false) {
    Carver c(workspace);
    void* h = c.take((size_t)(T * I) * 2);
    if (in_f16) {
        if (T <= SKINNY_MAX_T) {
            float* part = static_cast<float*>(c.take(0));
            hipError_t e = kind == TP_MLP_SWIGLU ? tpk::skinny_swiglu(X, W_gate, W_up, part, h, T, I, H, s, 1)
                                                 : tpk::skinny_linear(X, W_gate, part, T, I, H, H, h, I, 6, s, 1);
            if (e != hipSuccess) return e;
            return tpk::skinny_linear(h, W_down, part, T, H, I, I, Y, H, 0, s, 1);
        }
        void* split = c.take(0);
        const size_t split_bytes = need - c.off;
        hipError_t e = kind == TP_MLP_SWIGLU
                           ? tpk::gemm_f16_swiglu(X, W_gate, W_up, h, T, I, H, split, split_bytes, s)
                           : tpk::gemm_f16_store(X, W_gate, h, T, I, H, H, I, I, 1, 1, split, split_bytes, s);
        if (e != hipSuccess) return e;
        return tpk::gemm_f16_store(h, W_down, Y, T, H, I, I, H, H, 2, 0, split, split_bytes, s);
    }
    if (h_f16) {
        void* wd16 = c.take((size_t)(I * H) * 2);
        void* split = c.take(0);
        const size_t split_bytes = need - c.off;
        hipError_t e = kind == TP_MLP_SWIGLU
                           ? tpk::gemm_bf16_swiglu(X, W_gate, W_up, h, T, I, H, split, split_bytes, s, 1)
                           : tpk::gemm_bf16_store(X, W_gate, h, T, I, H, H, I, I, 1, 1, split, split_bytes, s);
        if (e == hipSuccess) e = tpk::bf16_to_f16(W_down, wd16, I * H, s);
        if (e != hipSuccess) return e;
        return tpk::gemm_f16_store(h, wd16, Y, T, H, I, I, H, H, 2, 0, split, split_bytes, s);
    }
    if (T <= SKINNY_MAX_T) {
        float* part = static_cast<float*>(c.take(0));
        hipError_t e = kind == TP_MLP_SWIGLU ? tpk::skinny_swiglu(X, W_gate, W_up, part, h, T, I, H, s)
                                             : tpk::skinny_linear(X, W_gate, part, T, I, H, H, h, I, 3, s);
        if (e != hipSuccess) return e;
        return tpk::skinny_linear(h, W_down, part, T, H, I, I, Y, H, 0, s);
    }
    void* split = c.take(0);
    const size_t split_bytes = need - c.off;
    hipError_t e = kind == TP_MLP_SWIGLU
                       ? tpk::gemm_bf16_swiglu(X, W_gate, W_up, h, T, I, H, split, split_bytes, s)
                       : tpk::gemm_bf16_store(X, W_gate, h, T, I, H, H, I, I, 0, 1, split, split_bytes, s);
    if (e != hipSuccess) return e;
    return tpk::gemm_bf16_store(h, W_down, Y, T, H, I, I, H, H, 2, 0, split, split_bytes, s);
}

tp_status tp_mlp_shard(const void* X, const void* W_gate, const void* W_up, const void* W_down,
                       float* Y_partial, int64_t T, int64_t H, int64_t I_shard, tp_mlp_kind kind,
                       tp_dtype in_dt, tp_dtype h_dt, void* workspace, size_t ws_bytes,
                       void* stream) {
    if (!X || !W_gate || !W_down || !Y_partial)
        return fail(TP_ERR_NULL_POINTER, "tp_mlp_shard: X, W_gate, W_down and Y_partial must be non-NULL");
    if (kind != TP_MLP_RELU && kind != TP_MLP_SWIGLU) return fail(TP_ERR_BAD_SHAPE, "tp_mlp_shard: unknown kind %d", (int)kind);
    if (kind == TP_MLP_SWIGLU && !W_up) return fail(TP_ERR_NULL_POINTER, "tp_mlp_shard: SwiGLU needs W_up");
    if (kind == TP_MLP_RELU && W_up) return fail(TP_ERR_BAD_SHAPE, "tp_mlp_shard: the ReLU form takes no W_up");
    if (T <= 0 || H <= 0 || I_shard <= 0)
        return fail(TP_ERR_BAD_SHAPE, "tp_mlp_shard: sizes must be positive (T=%lld H=%lld I=%lld)",
                    (long long)T, (long long)H, (long long)I_shard);
    if (in_dt == TP_F32 && h_dt != TP_F32) return fail(TP_ERR_BAD_DTYPE, "tp_mlp_shard: fp32 input keeps h in fp32");
    if (in_dt == TP_BF16 && h_dt != TP_BF16 && h_dt != TP_F16)
        return fail(TP_ERR_BAD_DTYPE, "tp_mlp_shard: bf16 input keeps h in bf16 or fp16");
    if (in_dt == TP_BF16 && h_dt == TP_F16 && T <= SKINNY_MAX_T)
        return fail(TP_ERR_UNSUPPORTED, "tp_mlp_shard: an fp16 h is offered for T > %d", (int)SKINNY_MAX_T);
    if (in_dt == TP_F16 && h_dt != TP_F16) return fail(TP_ERR_BAD_DTYPE, "tp_mlp_shard: fp16 input keeps h in fp16");
    if (in_dt != TP_F32 && in_dt != TP_BF16 && in_dt != TP_F16)
        return fail(TP_ERR_BAD_DTYPE, "tp_mlp_shard: input dtype %d not offered", (int)in_dt);
    if (in_dt == TP_F32 && kind == TP_MLP_SWIGLU) return fail(TP_ERR_UNSUPPORTED, "tp_mlp_shard: the fp32 path offers the ReLU form");
    const size_t need = tp_mlp_workspace_size(T, H, I_shard, kind, in_dt, h_dt);
    if (!workspace || ws_bytes < need)
        return fail(TP_ERR_WORKSPACE, "tp_mlp_shard: workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
    if (!aligned(workspace, 16)) return fail(TP_ERR_MISALIGNED, "tp_mlp_shard: workspace must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    if (in_dt == TP_F32) {
        if (!aligned(X, 4) || !aligned(W_gate, 4) || !aligned(W_down, 4) || !aligned(Y_partial, 4))
            return fail(TP_ERR_MISALIGNED, "tp_mlp_shard: fp32 pointers must be 4-byte aligned");
        float* h = static_cast<float*>(workspace);
        hipError_t e = tpk::gemm_f32(static_cast<const float*>(X), static_cast<const float*>(W_gate), h, T, I_shard,
                                     H, H, I_shard, I_shard, 1, 0, s);
        if (e != hipSuccess) return from_hip(e, "tp_mlp_shard");
        return from_hip(tpk::gemm_f32(h, static_cast<const float*>(W_down), Y_partial, T, H, I_shard, I_shard, H, H,
                                      0, 0, s),
                        "tp_mlp_shard");
    }
    if (!aligned(X, 16) || !aligned(W_gate, 16) || (W_up && !aligned(W_up, 16)) || !aligned(W_down, 16) ||
        !aligned(Y_partial, 16))
        return fail(TP_ERR_MISALIGNED, "tp_mlp_shard: 16-bit operands need 16-byte aligned pointers");
    if (H % 8 || I_shard % 8)
        return fail(TP_ERR_MISALIGNED, "tp_mlp_shard: 16-bit operands need H and I_shard multiples of 8");
    tp_status st = check_ld("tp_mlp_shard", "H", H);
    if (st == TP_OK) st = check_ld("tp_mlp_shard", "I_shard", I_shard);
    if (st != TP_OK) return st;
    return from_hip(mlp_bf16(X, W_gate, W_up, W_down, Y_partial, T, H, I_shard, kind, workspace, need, s,
                             in_dt == TP_BF16 && h_dt == TP_F16, in_dt == TP_F16),
                    "tp_mlp_shard");
}

size_t tp_mlp_fp8_workspace_size(int64_t T, int64_t H, int64_t I_shard, tp_mlp_kind kind) {
    if (T <= 0 || H <= 0 || I_shard <= 0) return 0;
    const size_t first = tpk::gemm_f8_split_bytes(T, I_shard, H, kind == TP_MLP_SWIGLU ? 1 : 0);
    const size_t second = tpk::gemm_f8_split_bytes(T, H, I_shard, 0);
    return round_up((size_t)(T * I_shard), WS_ALIGN) + round_up(first > second ? first : second, WS_ALIGN);
}

tp_status tp_mlp_shard_fp8(const void* X, const void* W_gate, const void* W_up, const void* W_down,
                           float* Y_partial, int64_t T, int64_t H, int64_t I_shard, tp_mlp_kind kind,
                           const tp_fp8_mlp_scales* q, void* workspace, size_t ws_bytes, void* stream) {
    const char* fn = "tp_mlp_shard_fp8";
    if (!X || !W_gate || !W_down || !Y_partial)
        return fail(TP_ERR_NULL_POINTER, "%s: X, W_gate, W_down and Y_partial must be non-NULL", fn);
    if (!q) return fail(TP_ERR_NULL_POINTER, "%s: scales q must be non-NULL", fn);
    if (kind != TP_MLP_RELU && kind != TP_MLP_SWIGLU) return fail(TP_ERR_BAD_SHAPE, "%s: unknown kind %d", fn, (int)kind);
    if (kind == TP_MLP_SWIGLU && !W_up) return fail(TP_ERR_NULL_POINTER, "%s: SwiGLU needs W_up", fn);
    if (kind == TP_MLP_RELU && W_up) return fail(TP_ERR_BAD_SHAPE, "%s: the ReLU form takes no W_up", fn);
    if (T <= 0 || H <= 0 || I_shard <= 0)
        return fail(TP_ERR_BAD_SHAPE, "%s: sizes must be positive (T=%lld H=%lld I=%lld)", fn, (long long)T,
                    (long long)H, (long long)I_shard);
    const bool up = kind == TP_MLP_SWIGLU;
    if (!(q->x_scale > 0.0f) || !(q->w_gate_scale > 0.0f) || !(q->w_down_scale > 0.0f) || !(q->h_scale > 0.0f) ||
        (up && !(q->w_up_scale > 0.0f)))
        return fail(TP_ERR_BAD_SHAPE, "%s: scales must be positive", fn);
    if (!aligned(X, 16) || !aligned(W_gate, 16) || (W_up && !aligned(W_up, 16)) || !aligned(W_down, 16) ||
        !aligned(Y_partial, 16))
        return fail(TP_ERR_MISALIGNED, "%s: fp8 path needs 16-byte aligned pointers", fn);
    if (H % 16 || I_shard % 16) return fail(TP_ERR_MISALIGNED, "%s: fp8 path needs H and I_shard multiples of 16", fn);
    tp_status st = check_ld(fn, "H", H);
    if (st == TP_OK) st = check_ld(fn, "I_shard", I_shard);
    if (st != TP_OK) return st;
    const size_t need = tp_mlp_fp8_workspace_size(T, H, I_shard, kind);
    st = check_ws(fn, workspace, ws_bytes, need);
    if (st != TP_OK) return st;
    hipStream_t s = as_stream(stream);
    Carver c(workspace);
    void* h = c.take((size_t)(T * I_shard));
    void* split = c.take(0);
    const size_t split_bytes = need - c.off;
    hipError_t e;
    if (up)
        e = tpk::gemm_f8_swiglu(X, W_gate, W_up, h, T, I_shard, H, q->x_scale * q->w_gate_scale,
                                q->x_scale * q->w_up_scale, q->h_scale, split, split_bytes, s);
    else
        e = tpk::gemm_f8_store(X, W_gate, h, T, I_shard, H, H, I_shard, I_shard, 4, 1,
                               q->x_scale * q->w_gate_scale, q->h_scale, split, split_bytes, s);
    if (e != hipSuccess) return from_hip(e, fn);
    return from_hip(tpk::gemm_f8_store(h, W_down, Y_partial, T, H, I_shard, I_shard, H, H, 2, 0,
                                       q->h_scale * q->w_down_scale, 1.0f, split, split_bytes, s),
                    fn);
}

// ---- attention shard --------------------------------------------------------------------------

static tp_status check_attn_desc(const tp_attn_desc* d, bool* decode) {
    if (!d) return fail(TP_ERR_NULL_POINTER, "tp_attn_shard: desc is NULL");
    if (d->B <= 0 || d->S <= 0 || d->H <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0)
        return fail(TP_ERR_BAD_SHAPE, "tp_attn_shard: B, S, H and head counts must be positive");
    if (d->head_dim != 128) return fail(TP_ERR_UNSUPPORTED, "tp_attn_shard: head_dim %d (only 128 is offered)", (int)d->head_dim);
    if (d->n_q_heads % d->n_kv_heads)
        return fail(TP_ERR_BAD_SHAPE, "tp_attn_shard: %d query heads do not group evenly over %d kv heads",
                    (int)d->n_q_heads, (int)d->n_kv_heads);
    if (d->causal != 1) return fail(TP_ERR_UNSUPPORTED, "tp_attn_shard: only causal attention is offered");
    if (!(d->rope_theta > 0.0f)) return fail(TP_ERR_BAD_SHAPE, "tp_attn_shard: rope_theta must be positive");
    if (d->H % 8) return fail(TP_ERR_MISALIGNED, "tp_attn_shard: H must be a multiple of 8");
    if (check_ld("tp_attn_shard", "H", d->H) != TP_OK) return TP_ERR_UNSUPPORTED;
    if (check_ld("tp_attn_shard", "n_q_heads * 128", (int64_t)d->n_q_heads * 128) != TP_OK) return TP_ERR_UNSUPPORTED;
    const bool has_cache = d->k_cache || d->v_cache;
    if (has_cache) {
        if (!d->k_cache || !d->v_cache) return fail(TP_ERR_NULL_POINTER, "tp_attn_shard: k_cache and v_cache go together");
        if (d->S != 1) return fail(TP_ERR_UNSUPPORTED, "tp_attn_shard: a KV cache is offered for S == 1 (decode) only");
        if (d->cache_len < 0 || d->cache_len >= d->cache_capacity)
            return fail(TP_ERR_BAD_SHAPE, "tp_attn_shard: need 0 <= cache_len (%lld) < cache_capacity (%lld)",
                        (long long)d->cache_len, (long long)d->cache_capacity);
        if (d->B > SKINNY_MAX_T) return fail(TP_ERR_UNSUPPORTED, "tp_attn_shard: decode offers at most %d sequences", (int)SKINNY_MAX_T);
        if (!aligned(d->k_cache, 16) || !aligned(d->v_cache, 16))
            return fail(TP_ERR_MISALIGNED, "tp_attn_shard: caches must be 16-byte aligned");
    } else if (d->S % 8) {
        return fail(TP_ERR_MISALIGNED, "tp_attn_shard: prefill needs S to be a multiple of 8 (S=%lld)", (long long)d->S);
    } else if (d->S > ((int64_t)1 << 24)) {
        return fail(TP_ERR_UNSUPPORTED, "tp_attn_shard: prefill offers S <= 2^24 (S=%lld)", (long long)d->S);
    } else if (d->B * d->S >= ((int64_t)1 << 31)) {
        return fail(TP_ERR_UNSUPPORTED, "tp_attn_shard: prefill offers fewer than 2^31 tokens (B*S=%lld)",
                    (long long)(d->B * d->S));
    }
    *decode = has_cache;
    return TP_OK;
}

static size_t attn_ws(const tp_attn_desc* d, bool decode, void* base, void** q, void** k,
                      void** vt, void** rope, void** att, void** part, size_t* split_bytes) {
    Carver c(base);
    const int64_t hq = d->n_q_heads, hkv = d->n_kv_heads;
    const int64_t nqkv = (hq + 2 * hkv) * 128;
    if (!decode) {
        const int64_t T = d->B * d->S;
        *rope = c.take((size_t)d->S * 64 * sizeof(float2));
        *q = c.take((size_t)(T * hq * 128) * 2);
        *k = c.take((size_t)(T * hkv * 128) * 2);
        *vt = c.take((size_t)(T * hkv * 128) * 2);
        *att = c.take((size_t)(T * hq * 128) * 2);
        const size_t s1 = tpk::gemm_bf16_split_bytes(T, nqkv, d->H, 0);
        const size_t s2 = tpk::gemm_bf16_split_bytes(T, d->H, hq * 128, 0);
        *split_bytes = s1 > s2 ? s1 : s2;
        *part = c.take(*split_bytes);
        return c.off;
    }
    const int64_t B = d->B;
    const size_t p1 = tpk::skinny_partials_bytes(B, nqkv, d->H);
    const size_t p2 = tpk::skinny_partials_bytes(B, d->H, hq * 128);
    *split_bytes = p1 > p2 ? p1 : p2;
    *part = c.take(*split_bytes);
    *att = c.take((size_t)(B * hq * 128) * 2);
    return c.off;
}

size_t tp_attn_workspace_size(const tp_attn_desc* desc, tp_dtype in_dt) {
    if (in_dt != TP_BF16) return 0;
    bool decode = false;
    if (check_attn_desc(desc, &decode) != TP_OK) return 0;
    void *q, *k, *vt, *rope, *att, *part;
    size_t split_bytes = 0;
    return attn_ws(desc, decode, nullptr, &q, &k, &vt, &rope, &att, &part, &split_bytes);
}

tp_status tp_attn_shard(const void* X, const void* W_qkv, const void* W_o, float* Y_partial,
                        const tp_attn_desc* desc, tp_dtype in_dt, void* workspace,
                        size_t ws_bytes, void* stream) {
    if (!X || !W_qkv || !W_o || !Y_partial)
        return fail(TP_ERR_NULL_POINTER, "tp_attn_shard: X, W_qkv, W_o and Y_partial must be non-NULL");
    bool decode = false;
    tp_status st = check_attn_desc(desc, &decode);
    if (st != TP_OK) return st;
    if (in_dt != TP_BF16) return fail(TP_ERR_BAD_DTYPE, "tp_attn_shard: the attention shard takes bf16 inputs");
    if (!aligned(X, 16) || !aligned(W_qkv, 16) || !aligned(W_o, 16) || !aligned(Y_partial, 16))
        return fail(TP_ERR_MISALIGNED, "tp_attn_shard: X, W_qkv, W_o and Y_partial must be 16-byte aligned");
    void *q, *k, *vt, *rope, *att, *part;
    size_t split_bytes = 0;
    const size_t need = attn_ws(desc, decode, nullptr, &q, &k, &vt, &rope, &att, &part, &split_bytes);
    if (!workspace || ws_bytes < need)
        return fail(TP_ERR_WORKSPACE, "tp_attn_shard: workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
    if (!aligned(workspace, 16)) return fail(TP_ERR_MISALIGNED, "tp_attn_shard: workspace must be 16-byte aligned");
    attn_ws(desc, decode, workspace, &q, &k, &vt, &rope, &att, &part, &split_bytes);
    hipStream_t s = as_stream(stream);
    const int hq = desc->n_q_heads, hkv = desc->n_kv_heads;
    const int64_t H = desc->H, dq = (int64_t)hq * 128;
    if (!decode) {
        const int64_t T = desc->B * desc->S;
        hipError_t e = tpk::rope_table(static_cast<float2*>(rope), 0, desc->S, desc->rope_theta, s);
        if (e != hipSuccess) return from_hip(e, "tp_attn_shard");
        tpk::QKVOut o{q, k, vt, static_cast<const float2*>(rope), desc->B, desc->S, hq, hkv};
        e = tpk::gemm_bf16_qkv_rope(X, W_qkv, H, o, part, split_bytes, s);
        if (e != hipSuccess) return from_hip(e, "tp_attn_shard");
        e = tpk::flash_attn_fwd(q, k, vt, att, desc->B, desc->S, hq, hkv, s);
        if (e != hipSuccess) return from_hip(e, "tp_attn_shard");
        return from_hip(tpk::gemm_bf16_store(att, W_o, Y_partial, T, H, dq, dq, H, H, 2, 0, part, split_bytes, s),
                        "tp_attn_shard");
    }
    const int64_t B = desc->B;
    hipError_t e = tpk::decode_attn_step(X, W_qkv, static_cast<float*>(part), B, H, hq, hkv, desc->cache_len,
                                         desc->rope_theta, desc->k_cache, desc->v_cache, desc->cache_capacity,
                                         att, s);
    if (e != hipSuccess) return from_hip(e, "tp_attn_shard");
    return from_hip(tpk::skinny_linear(att, W_o, static_cast<float*>(part), B, H, dq, dq, Y_partial, H, 0, s),
                    "tp_attn_shard");
}

// ---- the whole decode step -------------------------------------------------------------------

static tp_status check_decode_step(const tp_attn_desc* d, int64_t I, int64_t V, bool has_lm) {
    const char* fn = "tp_decode_step";
    bool decode = false;
    tp_status st = check_attn_desc(d, &decode);
    if (st != TP_OK) return st;
    if (!decode) return fail(TP_ERR_BAD_SHAPE, "%s: desc must describe a decode step (S == 1 with k_cache and v_cache)", fn);
    if (I <= 0 || V < 0) return fail(TP_ERR_BAD_SHAPE, "%s: need I_shard > 0 and V_shard >= 0", fn);
    if ((V > 0) != has_lm) return fail(TP_ERR_BAD_SHAPE, "%s: W_lm and V_shard > 0 go together", fn);
    if (I % 8 || V % 8) return fail(TP_ERR_MISALIGNED, "%s: I_shard and V_shard must be multiples of 8", fn);
    if (check_ld(fn, "I_shard", I) != TP_OK) return TP_ERR_UNSUPPORTED;
    return TP_OK;
}

size_t tp_decode_step_workspace_size(const tp_attn_desc* desc, int64_t I_shard, int64_t V_shard) {
    if (!desc || check_decode_step(desc, I_shard, V_shard, V_shard > 0) != TP_OK) return 0;
    return round_up(tpk::decode_step_ws_bytes(desc->B, desc->H, desc->n_q_heads, desc->n_kv_heads, I_shard, V_shard),
                    WS_ALIGN);
}

static tp_status decode_step_impl(const char* fn, bool packed, const void* X, const void* W_qkv, const void* W_o,
                                  const tp_attn_desc* desc, const void* W_gate, const void* W_up, const void* W_down,
                                  int64_t I_shard, const void* W_lm, int64_t V_shard, float* Y_attn, float* Y_mlp,
                                  float* logits, void* workspace, size_t ws_bytes, void* stream) {
    if (!X || !W_qkv || !W_o || !W_gate || !W_up || !W_down || !Y_attn || !Y_mlp)
        return fail(TP_ERR_NULL_POINTER, "%s: X, the attention and MLP weights, Y_attn and Y_mlp must be non-NULL", fn);
    if (V_shard > 0 && !logits) return fail(TP_ERR_NULL_POINTER, "%s: logits must be non-NULL when V_shard > 0", fn);
    tp_status st = check_decode_step(desc, I_shard, V_shard, W_lm != nullptr);
    if (st != TP_OK) return st;
    const void* ptrs[] = {X, W_qkv, W_o, W_gate, W_up, W_down, Y_attn, Y_mlp};
    for (const void* q : ptrs)
        if (!aligned(q, 16)) return fail(TP_ERR_MISALIGNED, "%s: tensors must be 16-byte aligned", fn);
    if (V_shard > 0 && (!aligned(W_lm, 16) || !aligned(logits, 16)))
        return fail(TP_ERR_MISALIGNED, "%s: W_lm and logits must be 16-byte aligned", fn);
    st = check_ws(fn, workspace, ws_bytes, tp_decode_step_workspace_size(desc, I_shard, V_shard));
    if (st != TP_OK) return st;
    return from_hip(tpk::decode_step(X, W_qkv, W_o, W_gate, W_up, W_down, W_lm, desc->B, desc->H, desc->n_q_heads,
                                     desc->n_kv_heads, I_shard, V_shard, desc->cache_len, desc->rope_theta,
                                     desc->k_cache, desc->v_cache, desc->cache_capacity, Y_attn, Y_mlp,
                                     V_shard > 0 ? logits : nullptr, workspace, as_stream(stream), packed),
                    fn);
}

tp_status tp_decode_step(const void* X, const void* W_qkv, const void* W_o, const tp_attn_desc* desc,
                         const void* W_gate, const void* W_up, const void* W_down, int64_t I_shard,
                         const void* W_lm, int64_t V_shard, float* Y_attn, float* Y_mlp, float* logits,
                         void* workspace, size_t ws_bytes, void* stream) {
    return decode_step_impl("tp_decode_step", false, X, W_qkv, W_o, desc, W_gate, W_up, W_down, I_shard, W_lm,
                            V_shard, Y_attn, Y_mlp, logits, workspace, ws_bytes, stream);
}

tp_status tp_decode_step_packed(const void* X, const void* W_qkv, const void* W_o, const tp_attn_desc* desc,
                                const void* W_gate, const void* W_up, const void* W_down, int64_t I_shard,
                                const void* W_lm, int64_t V_shard, float* Y_attn, float* Y_mlp, float* logits,
                                void* workspace, size_t ws_bytes, void* stream) {
    return decode_step_impl("tp_decode_step_packed", true, X, W_qkv, W_o, desc, W_gate, W_up, W_down, I_shard,
                            W_lm, V_shard, Y_attn, Y_mlp, logits, workspace, ws_bytes, stream);
}

// packed weights are limited to 2^36 elements (padded), which keeps the copy's grid below 2^25
// workgroups and every index in 64 bits
static bool packable(int64_t K, int64_t N) {
    if (K <= 0 || N <= 0 || K >= ((int64_t)1 << 36) || N >= ((int64_t)1 << 36)) return false;
    const int64_t strips = (N + 127) / 128;
    return strips <= (((int64_t)1 << 36) / 128) / K;
}

size_t tp_packed_strips_bytes(int64_t K, int64_t N) {
    if (N % 8 || !packable(K, N)) return 0;
    return tpk::packed_strips_bytes(K, N);
}

tp_status tp_pack_strips(const void* W, int64_t K, int64_t N, void* W_packed, void* stream) {
    const char* fn = "tp_pack_strips";
    if (!W || !W_packed) return fail(TP_ERR_NULL_POINTER, "%s: W and W_packed must be non-NULL", fn);
    if (K <= 0 || N <= 0) return fail(TP_ERR_BAD_SHAPE, "%s: need K > 0 and N > 0", fn);
    if (N % 8) return fail(TP_ERR_MISALIGNED, "%s: N must be a multiple of 8", fn);
    if (!packable(K, N))
        return fail(TP_ERR_UNSUPPORTED, "%s: K x N (N rounded up to 128) must be at most 2^36 elements", fn);
    if (!aligned(W, 16) || !aligned(W_packed, 16))
        return fail(TP_ERR_MISALIGNED, "%s: W and W_packed must be 16-byte aligned", fn);
    return from_hip(tpk::pack_strips(W, K, N, W_packed, as_stream(stream)), fn);
}

// ---- merges ------------------------------------------------------------------------------------

tp_status tp_partial_sum(const float* const* partials, int32_t k, float* out, int64_t n_elems,
                         void* stream) {
    if (!partials || !out) return fail(TP_ERR_NULL_POINTER, "tp_partial_sum: partials and out must be non-NULL");
    if (k < 1 || k > 16) return fail(TP_ERR_BAD_SHAPE, "tp_partial_sum: k=%d outside 1..16", (int)k);
    if (n_elems <= 0) return fail(TP_ERR_BAD_SHAPE, "tp_partial_sum: n_elems must be positive");
    if (!aligned(out, 16)) return fail(TP_ERR_MISALIGNED, "tp_partial_sum: out must be 16-byte aligned");
    for (int i = 0; i < k; ++i) {
        if (!partials[i]) return fail(TP_ERR_NULL_POINTER, "tp_partial_sum: partials[%d] is NULL", i);
        if (!aligned(partials[i], 16)) return fail(TP_ERR_MISALIGNED, "tp_partial_sum: partials[%d] must be 16-byte aligned", i);
    }
    return from_hip(tpk::partial_sum(partials, k, out, n_elems, as_stream(stream)), "tp_partial_sum");
}

// ---- MoE MLP shard ----------------------------------------------------------------------

static bool moe_offsets_ok(const int64_t* offs, int32_t E) {
    if (!offs || offs[0] != 0) return false;
    for (int32_t e = 0; e < E; ++e)
        if (offs[e + 1] < offs[e]) return false;
    return offs[E] < ((int64_t)1 << 31);
}

static int64_t moe_max_rows(const int64_t* offs, int32_t E) {
    int64_t m = 0;
    for (int32_t e = 0; e < E; ++e) m = offs[e + 1] - offs[e] > m ? offs[e + 1] - offs[e] : m;
    return m;
}

// Experts of at most SKINNY_MAX_T rows each run one after another through the weight-streaming
// kernels; otherwise all experts share one grouped gate/up launch and one grouped down launch.
size_t tp_moe_workspace_size(int64_t T, int64_t H, int64_t I_shard, int32_t E, const int64_t* expert_offsets) {
    if (T <= 0 || H <= 0 || I_shard <= 0 || E < 1 || E > 1024 || !moe_offsets_ok(expert_offsets, E)) return 0;
    const int64_t R = expert_offsets[E];
    const size_t rows = round_up((size_t)(R * H) * 2, WS_ALIGN) + round_up((size_t)(R * H) * 4, WS_ALIGN);
    if (moe_max_rows(expert_offsets, E) > SKINNY_MAX_T) {
        const size_t gu = tpk::gemm_bf16_grouped_split_bytes(expert_offsets, E, I_shard, H, 1);
        const size_t dn = tpk::gemm_bf16_grouped_split_bytes(expert_offsets, E, H, I_shard, 0);
        // Xg and h each get one more row, of zeros (moe_zero_rows)
        return rows + round_up((size_t)H * 2, WS_ALIGN) + round_up((size_t)((R + 1) * I_shard) * 2, WS_ALIGN) +
               round_up(gu > dn ? gu : dn, WS_ALIGN);
    }
    size_t mlp = 0;
    for (int32_t e = 0; e < E; ++e) {
        const int64_t n = expert_offsets[e + 1] - expert_offsets[e];
        if (n > 0) {
            const size_t b = tp_mlp_workspace_size(n, H, I_shard, TP_MLP_SWIGLU, TP_BF16, TP_BF16);
            mlp = b > mlp ? b : mlp;
        }
    }
    return rows + mlp;
}

tp_status tp_moe_mlp_shard(const void* X, int64_t T, int64_t H, int64_t I_shard, int32_t E, const void* W_gate,
                           const void* W_up, const void* W_down, const int64_t* expert_offsets,
                           const int32_t* row_token, int32_t k, const int32_t* token_rows, const float* gates,
                           float* Y_partial, void* workspace, size_t ws_bytes, void* stream) {
    const char* fn = "tp_moe_mlp_shard";
    if (!X || !W_gate || !W_up || !W_down || !expert_offsets || !token_rows || !gates || !Y_partial)
        return fail(TP_ERR_NULL_POINTER, "%s: X, the weights, expert_offsets, token_rows, gates and Y_partial must be "
                                         "non-NULL", fn);
    if (T <= 0 || H <= 0 || I_shard <= 0)
        return fail(TP_ERR_BAD_SHAPE, "%s: sizes must be positive (T=%lld H=%lld I=%lld)", fn, (long long)T,
                    (long long)H, (long long)I_shard);
    if (E < 1 || E > 1024) return fail(TP_ERR_BAD_SHAPE, "%s: E=%d outside 1..1024", fn, (int)E);
    if (k < 1 || k > 16) return fail(TP_ERR_BAD_SHAPE, "%s: k=%d outside 1..16", fn, (int)k);
    if (T >= ((int64_t)1 << 31)) return fail(TP_ERR_UNSUPPORTED, "%s: T=%lld tokens (at most 2^31 - 1)", fn, (long long)T);
    if (!moe_offsets_ok(expert_offsets, E))
        return fail(TP_ERR_BAD_SHAPE, "%s: expert_offsets must start at 0, not decrease, and end below 2^31", fn);
    const int64_t R = expert_offsets[E];
    if (R > 0 && !row_token) return fail(TP_ERR_NULL_POINTER, "%s: row_token must be non-NULL when rows exist", fn);
    if (H % 8 || I_shard % 8) return fail(TP_ERR_MISALIGNED, "%s: H and I_shard must be multiples of 8", fn);
    if (check_ld(fn, "H", H) != TP_OK || check_ld(fn, "I_shard", I_shard) != TP_OK) return TP_ERR_UNSUPPORTED;
    if (!aligned(X, 16) || !aligned(W_gate, 16) || !aligned(W_up, 16) || !aligned(W_down, 16) || !aligned(Y_partial, 16))
        return fail(TP_ERR_MISALIGNED, "%s: X, the weights and Y_partial must be 16-byte aligned", fn);
    if ((row_token && !aligned(row_token, 4)) || !aligned(token_rows, 4) || !aligned(gates, 4))
        return fail(TP_ERR_MISALIGNED, "%s: row_token, token_rows and gates must be 4-byte aligned", fn);
    if (moe_max_rows(expert_offsets, E) > SKINNY_MAX_T) {
        // grouped launches number their 256-row x 128-column tiles in 32 bits (with up to 4
        // tail pieces each): keep every launch far below that
        int64_t row_tiles = 0;
        for (int32_t x = 0; x < E; ++x) row_tiles += (expert_offsets[x + 1] - expert_offsets[x] + 255) / 256;
        const int64_t col_tiles = ((H > I_shard ? H : I_shard) + 127) / 128;
        if (row_tiles * col_tiles >= ((int64_t)1 << 28))
            return fail(TP_ERR_UNSUPPORTED, "%s: %lld row tiles x %lld column tiles exceed the grouped GEMM's 2^28 tiles",
                        fn, (long long)row_tiles, (long long)col_tiles);
    }
    const size_t need = tp_moe_workspace_size(T, H, I_shard, E, expert_offsets);
    tp_status st = check_ws(fn, workspace, ws_bytes, need);
    if (st != TP_OK) return st;
    hipStream_t s = as_stream(stream);
    Carver c(workspace);
    if (moe_max_rows(expert_offsets, E) > SKINNY_MAX_T) {
        // grouped launches: the rows of an expert's last tile past its end read a row of zeros
        // (row R of Xg, row R of h) rather than a copy of a real row; zero operands draw less
        // power at the same speed. The DMA offsets of those rows (up to (R + 1) rows) are 32-bit.
        void* Xg = c.take((size_t)((R + 1) * H) * 2);
        float* Yg = static_cast<float*>(c.take((size_t)(R * H) * 4));
        void* h = c.take((size_t)((R + 1) * I_shard) * 2);
        void* split = c.take(0);
        const size_t split_bytes = need - c.off;
        const bool zr = (R + 1) * (H > I_shard ? H : I_shard) < ((int64_t)1 << 31);
        unsigned char* xz = static_cast<unsigned char*>(Xg) + (size_t)(R * H) * 2;
        unsigned char* hz = static_cast<unsigned char*>(h) + (size_t)(R * I_shard) * 2;
        hipError_t e = tpk::moe_gather(X, row_token, Xg, R, T, H, s, zr ? xz : nullptr, H, zr ? hz : nullptr, I_shard);
        if (e == hipSuccess)
            e = tpk::gemm_bf16_swiglu_grouped(Xg, W_gate, W_up, h, expert_offsets, E, I_shard, H, split, split_bytes, s,
                                              zr ? R : -1);
        if (e == hipSuccess)
            e = tpk::gemm_bf16_f32out_grouped(h, W_down, Yg, expert_offsets, E, H, I_shard, split, split_bytes, s,
                                              zr ? R : -1);
        if (e == hipSuccess) e = tpk::moe_combine(Yg, token_rows, gates, k, Y_partial, T, R, H, s);
        return from_hip(e, fn);
    }
    void* Xg = c.take((size_t)(R * H) * 2);
    float* Yg = static_cast<float*>(c.take((size_t)(R * H) * 4));
    hipError_t e = tpk::moe_gather(X, row_token, Xg, R, T, H, s);
    void* mlp_ws = c.take(0);   // the largest expert's MLP workspace, reused expert after expert
    for (int32_t x = 0; x < E && e == hipSuccess; ++x) {
        const int64_t a = expert_offsets[x], n = expert_offsets[x + 1] - a;
        if (n == 0) continue;
        const size_t wo = (size_t)(x * H * I_shard) * 2;
        e = mlp_bf16(static_cast<const unsigned char*>(Xg) + (size_t)(a * H) * 2,
                     static_cast<const unsigned char*>(W_gate) + wo, static_cast<const unsigned char*>(W_up) + wo,
                     static_cast<const unsigned char*>(W_down) + wo, Yg + a * H, n, H, I_shard, TP_MLP_SWIGLU,
                     mlp_ws, tp_mlp_workspace_size(n, H, I_shard, TP_MLP_SWIGLU, TP_BF16, TP_BF16), s);
    }
    if (e == hipSuccess) e = tpk::moe_combine(Yg, token_rows, gates, k, Y_partial, T, R, H, s);
    return from_hip(e, fn);
}

size_t tp_linear_backward_workspace_size(int64_t T, int64_t K, int64_t N) {
    if (T <= 0 || K <= 0 || N <= 0) return 0;
    return round_up(tpk::linear_backward_ws_bytes(T, K, N), WS_ALIGN);
}

tp_status tp_linear_backward(const void* X, const void* W_shard, const void* dY, float* dX, float* dW,
                             int64_t T, int64_t K, int64_t N, tp_dtype in_dt, void* workspace,
                             size_t ws_bytes, void* stream) {
    const char* fn = "tp_linear_backward";
    if (!X || !W_shard || !dY || !dX || !dW)
        return fail(TP_ERR_NULL_POINTER, "%s: X, W_shard, dY, dX and dW must be non-NULL", fn);
    if (in_dt != TP_BF16) return fail(TP_ERR_BAD_DTYPE, "%s: input dtype %d not offered (bf16 only)", fn, (int)in_dt);
    if (T <= 0 || K <= 0 || N <= 0)
        return fail(TP_ERR_BAD_SHAPE, "%s: sizes must be positive (T=%lld K=%lld N=%lld)", fn, (long long)T,
                    (long long)K, (long long)N);
    if (T % 8 || K % 8 || N % 8)
        return fail(TP_ERR_MISALIGNED, "%s: T, K and N must be multiples of 8 (T=%lld K=%lld N=%lld)", fn,
                    (long long)T, (long long)K, (long long)N);
    if (T >= ((int64_t)1 << 23) || K >= ((int64_t)1 << 23) || N >= ((int64_t)1 << 23))
        return fail(TP_ERR_UNSUPPORTED, "%s: T, K and N must be below 2^23", fn);
    // the two GEMMs launch one 256-thread workgroup per 256 x 256 output tile (up to 4 per tile
    // with the tail split); a grid holds fewer than 2^32 threads, so the tiles stay below 2^22
    if (((T + 255) / 256) * ((K + 255) / 256) + ((K + 255) / 256) * ((N + 255) / 256) >= ((int64_t)1 << 22))
        return fail(TP_ERR_UNSUPPORTED, "%s: dX and dW need fewer than 2^22 tiles of 256 x 256", fn);
    if (!aligned(X, 16) || !aligned(W_shard, 16) || !aligned(dY, 16) || !aligned(dX, 16) || !aligned(dW, 16))
        return fail(TP_ERR_MISALIGNED, "%s: X, W_shard, dY, dX and dW must be 16-byte aligned", fn);
    tp_status st = check_ws(fn, workspace, ws_bytes, tp_linear_backward_workspace_size(T, K, N));
    if (st != TP_OK) return st;
    return from_hip(tpk::linear_backward(X, W_shard, dY, dX, dW, T, K, N, workspace, as_stream(stream)), fn);
}

tp_status tp_merge_rmsnorm(const float* const* partials, int32_t k, const void* residual, const void* gamma,
                           float eps, void* residual_out, void* normed, int64_t T, int64_t H, void* stream) {
    const char* fn = "tp_merge_rmsnorm";
    if (!partials || !residual || !gamma || !residual_out || !normed)
        return fail(TP_ERR_NULL_POINTER, "%s: partials, residual, gamma, residual_out and normed must be non-NULL", fn);
    if (k < 1 || k > 16) return fail(TP_ERR_BAD_SHAPE, "%s: k=%d outside 1..16", fn, (int)k);
    if (T <= 0 || H <= 0) return fail(TP_ERR_BAD_SHAPE, "%s: T and H must be positive (T=%lld H=%lld)", fn,
                                      (long long)T, (long long)H);
    if (T >= ((int64_t)1 << 31)) return fail(TP_ERR_UNSUPPORTED, "%s: T=%lld rows (at most 2^31 - 1)", fn, (long long)T);
    if (H % 8 || H > 16384)
        return fail(TP_ERR_UNSUPPORTED, "%s: H=%lld (a multiple of 8, at most 16384)", fn, (long long)H);
    if (!(eps >= 0.0f) || !(eps <= 1e30f)) return fail(TP_ERR_BAD_SHAPE, "%s: eps must be finite and >= 0", fn);
    if (!aligned(residual, 16) || !aligned(gamma, 16) || !aligned(residual_out, 16) || !aligned(normed, 16))
        return fail(TP_ERR_MISALIGNED, "%s: residual, gamma, residual_out and normed must be 16-byte aligned", fn);
    for (int i = 0; i < k; ++i) {
        if (!partials[i]) return fail(TP_ERR_NULL_POINTER, "%s: partials[%d] is NULL", fn, i);
        if (!aligned(partials[i], 16)) return fail(TP_ERR_MISALIGNED, "%s: partials[%d] must be 16-byte aligned", fn, i);
    }
    return from_hip(tpk::merge_rmsnorm(partials, k, residual, gamma, eps, residual_out, normed, T, H,
                                       as_stream(stream)), fn);
}

}  // extern "C"
