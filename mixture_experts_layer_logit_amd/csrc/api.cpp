// Host side of the C ABI declared in include/moe.h: argument checks, workspace
// layout and the launch sequence of the MoE-layer forward.  Nothing here
// allocates device memory, copies to the host or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "moe.h"

extern "C" {
hipError_t moe_launch_gate(int dtype, const void* x, const void* Wg, const float* bg, float* logits, int T, int d,
                           int E, hipStream_t stream);
hipError_t moe_launch_gate_route(int dtype, const void* x, const void* Wg, const float* bg, float* logits, int T,
                                 int d, int E, int k, int normalize, float lambda, int32_t* topk_idx, float* topk_w,
                                 hipStream_t stream);
hipError_t moe_launch_router(const float* logits, int T, int E, int k, int normalize, float lambda,
                             int32_t* topk_idx, float* topk_w, hipStream_t stream);
hipError_t moe_launch_permute(int dtype, const int32_t* topk_idx, const void* x, int T, int d, int E, int k,
                              long long C, int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* src_token,
                              void* x_perm, int32_t* chunk_cnt, hipStream_t stream);
hipError_t moe_launch_grouped_gemm(int dtype, int epi, const void* A, const int32_t* gather, int gather_rows,
                                   const void* W, void* C, const int32_t* offsets, int E, int K, int Nw, int Nout,
                                   int F, int max_rows, int mean_rows, int ncu, float* partial, const void* aux_in,
                                   void* aux_out, int aux_ld, hipStream_t stream);
size_t moe_grouped_gemm_partial_bytes(int dtype, int mean_rows);
hipError_t moe_launch_combine(int dtype, const void* y_perm, const int32_t* slot, const float* topk_w,
                              const void* y_add, int T, int d, int k, int max_rows, void* y, hipStream_t stream);
size_t moe_router_stats_partial_bytes(int T, int E);
hipError_t moe_launch_combine_bwd(int dtype, const void* dy, const void* y_perm, const int32_t* slot,
                                  const float* topk_w, int T, int d, int k, int max_rows, void* d_yp, float* d_w,
                                  hipStream_t stream);
hipError_t moe_launch_router_bwd(const float* logits, const int32_t* topk_idx, const int32_t* slot, const float* d_w,
                                 int T, int E, int k, int normalize, float lambda, float aux_coef, float z_coef,
                                 const int32_t* counts, float* dz, hipStream_t stream);
hipError_t moe_launch_kofs(const int32_t* offsets, int E, int max_rows, int align, int32_t* kofs, hipStream_t stream);
hipError_t moe_launch_transpose(int dtype, const void* src, int B, int R, int C, void* dst, hipStream_t stream);
hipError_t moe_launch_seg_transpose(int dtype, const void* src, const int32_t* gather, int gather_rows,
                                    const int32_t* offsets, const int32_t* kofs, int E, int max_rows, int C, int ld,
                                    void* dst, hipStream_t stream);
hipError_t moe_launch_unpermute_bwd(int dtype, const void* dx_perm, const int32_t* slot, int T, int d, int k,
                                    int max_rows, const float* dz, const void* Wg, int E, void* dx, hipStream_t stream);
size_t moe_gate_wgrad_partial_bytes(int T, int d, int E);
hipError_t moe_launch_zero(float* p, size_t n, hipStream_t stream);
hipError_t moe_launch_gate_wgrad(int dtype, const float* dz, const void* x, int T, int d, int E, float* partial,
                                 float* dWg, float* dbg, hipStream_t stream);
hipError_t moe_launch_grouped_gemm_wt(int epi, const void* A, const void* W, void* C, const int32_t* offsets, int E,
                                      int K, int Nw, int Nout, int F, int max_rows, int mean_rows, int ncu,
                                      float* partial, const void* aux_in, int aux_ld, hipStream_t stream);
hipError_t moe_launch_grouped_gemm_kgrp(int dtype, const void* A, const void* W, float* C, const int32_t* kofs, int E,
                                        int lda, int M, int N, int ncu, hipStream_t stream);
hipError_t moe_launch_quantize_fp8(int dtype, const void* src, long long R, int K, uint8_t* codes, float* scales,
                                   hipStream_t stream);
hipError_t moe_launch_grouped_gemm_fp8(int epi, const void* A, const int32_t* gather, int gather_rows, const void* W,
                                       void* C, const int32_t* offsets, int E, int K, int Nw, int Nout, int F,
                                       int max_rows, int mean_rows, int ncu, float* partial, const float* a_scale,
                                       const float* w_scale, hipStream_t stream);
hipError_t moe_launch_router_stats(const float* logits, int T, int E, int k, int normalize, float lambda,
                                   const int32_t* counts, const int32_t* offsets, double* partial, float* frac,
                                   float* mean_prob, float* scalars, hipStream_t stream);
}

namespace {

constexpr int kChunk = 256;      // tokens per permutation chunk (matches the permute kernels)
constexpr int kMaxE = 1024;
constexpr int kMaxK = 8;
constexpr int kMaxT = 1 << 24;
constexpr int kMaxDim = 65536;
constexpr size_t kAlign = 256;
// The fused row gather of the up projection addresses x with 32-bit byte
// offsets, and offsets from 0xF0000000 up are its out-of-range marker.
constexpr unsigned long long kGatherBytes = 0xF0000000ull;

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

moe_status ok()
{
    g_err[0] = 0;
    return MOE_OK;
}

size_t elem_bytes(const moe_problem* p) { return p->dtype == MOE_F32 ? 4 : 2; }
int n1_of(const moe_problem* p) { return p->act == MOE_ACT_SWIGLU ? 2 * p->F : p->F; }

long long capacity_of(const moe_problem* p)
{
    const double cf = p->capacity_factor;
    if (!(cf > 0.0))
        return -1;
    return (long long)std::ceil(cf * p->T * p->k / p->E);
}

moe_status check_problem(const moe_problem* p)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "problem is NULL");
    if (p->T < 0 || p->T > kMaxT)
        return fail(p->T < 0 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED, "T=%d outside [0, %d]", p->T, kMaxT);
    if (p->E < 1 || p->E > kMaxE)
        return fail(p->E < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED, "E=%d outside [1, %d]", p->E, kMaxE);
    if (p->k < 1 || p->k > p->E)
        return fail(MOE_ERR_INVALID_ARG, "k=%d outside [1, E=%d]", p->k, p->E);
    if (p->k > kMaxK)
        return fail(MOE_ERR_UNSUPPORTED, "k=%d above %d", p->k, kMaxK);
    if (p->d < 64 || p->d > kMaxDim || p->d % 64)
        return fail(MOE_ERR_UNSUPPORTED, "d=%d must be a multiple of 64 in [64, %d]", p->d, kMaxDim);
    if (p->F < 64 || p->F > kMaxDim || p->F % 64)
        return fail(MOE_ERR_UNSUPPORTED, "F=%d must be a multiple of 64 in [64, %d]", p->F, kMaxDim);
    if (p->act != MOE_ACT_RELU && p->act != MOE_ACT_SWIGLU)
        return fail(MOE_ERR_INVALID_ARG, "act=%d is neither MOE_ACT_RELU nor MOE_ACT_SWIGLU", p->act);
    if (p->dtype != MOE_F32 && p->dtype != MOE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "dtype=%d is neither MOE_F32 nor MOE_BF16", p->dtype);
    if (p->normalize != 0 && p->normalize != 1)
        return fail(MOE_ERR_INVALID_ARG, "normalize=%d is neither 0 nor 1", p->normalize);
    if (p->normalize && !(std::isfinite(p->lambda) && p->lambda > 0.0f))
        return fail(MOE_ERR_INVALID_ARG, "lambda=%g must be finite and > 0 with normalisation", (double)p->lambda);
    if (std::isnan(p->capacity_factor) || std::isinf(p->capacity_factor))
        return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite");
    const long long rows = (long long)p->T * p->k;
    if (rows * (long long)std::max(n1_of(p), p->d) >= (1LL << 40))
        return fail(MOE_ERR_UNSUPPORTED, "problem too large");
    // one expert's weight matrix is addressed with 32-bit byte offsets
    if ((long long)n1_of(p) * p->d * (long long)elem_bytes(p) >= (1LL << 31) ||
        (long long)p->d * p->F * (long long)elem_bytes(p) >= (1LL << 31))
        return fail(MOE_ERR_UNSUPPORTED, "one expert's weights must stay below 2 GiB");
    return MOE_OK;
}

moe_status check_ptr(const void* ptr, const char* name, size_t align)
{
    if (!ptr)
        return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
    if (reinterpret_cast<uintptr_t>(ptr) % align)
        return fail(MOE_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
    return MOE_OK;
}

#define CHECK(expr)                     \
    do {                                \
        moe_status _s = (expr);         \
        if (_s != MOE_OK)               \
            return _s;                  \
    } while (0)

// Whether x is small enough to be read through src_token by the up projection.
bool gather_ok(const moe_problem* p)
{
    return (unsigned long long)p->T * p->d * elem_bytes(p) < kGatherBytes;
}

// Workspace layout of a problem: every piece 256-byte aligned.  x_perm is
// only there (non-zero size) when x is too large to gather from directly.
struct Layout {
    size_t topk_idx, topk_w, counts, offsets, slot, src_token, chunk_cnt, logits, stats, partial, h, y_perm, x_perm,
        total;
};

int mean_rows_of(const moe_problem* p);

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// with_partial: room for the K-split partial tiles of the grouped GEMM's last
// round (without it the GEMMs run unsplit).
Layout layout_of(const moe_problem* p, bool with_partial = true)
{
    Layout L;
    const size_t T = (size_t)p->T, k = (size_t)p->k, E = (size_t)p->E, d = (size_t)p->d, F = (size_t)p->F;
    const size_t b = elem_bytes(p);
    const size_t nchunks = (T + kChunk - 1) / kChunk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += round_up(bytes);
        return at;
    };
    L.topk_idx = take(T * k * 4);
    L.topk_w = take(T * k * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.slot = take(T * k * 4);
    L.src_token = take(T * k * 4);
    L.chunk_cnt = take(std::max<size_t>(nchunks, 1) * E * 4);
    L.logits = take(T * E * 4);
    L.stats = take(moe_router_stats_partial_bytes(p->T, p->E));
    L.partial = take(with_partial ? moe_grouped_gemm_partial_bytes(p->dtype, mean_rows_of(p)) : 0);
    L.h = take(T * k * F * b);
    L.y_perm = take(T * k * d * b);
    L.x_perm = take(gather_ok(p) ? 0 : T * k * d * b);
    L.total = off;
    return L;
}

template <typename Tp>
Tp* at(void* ws, size_t off)
{
    return reinterpret_cast<Tp*>(static_cast<char*>(ws) + off);
}

int cu_count()
{
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

moe_status hip_status(hipError_t e, const char* what)
{
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

// ---- the allocation-free forward's scratch
// One file-scope device array per GPU (each device holds its own copy, at its
// own address, from the library's load until the process ends).  Host code
// never uses the array's name as an address: it takes the device address
// once per device with hipGetSymbolAddress and passes that to the kernels.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of this device's scratch (looked up on the device's first
// call, with the device current).
moe_status scratch_address(void** out)
{
    static std::mutex mu;
    static void* addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64)
        return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the 64 the scratch table holds", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        addr[dev] = ptr;
    }
    *out = addr[dev];
    return MOE_OK;
}

moe_status check_ws(const moe_problem* p, const void* ws, size_t ws_bytes)
{
    const size_t need = layout_of(p).total;
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, need);
    return check_ptr(ws, "ws", 16);
}

// ---- the steps, on validated arguments
moe_status do_route(const moe_problem* p, const void* x, const void* Wg, const float* bg, float* logits,
                    int32_t* topk_idx, float* topk_w, hipStream_t s)
{
    // up to 64 experts one kernel computes the logits and routes them
    if (Wg && p->E <= 64)
        return hip_status(moe_launch_gate_route(p->dtype, x, Wg, bg, logits, p->T, p->d, p->E, p->k, p->normalize,
                                                p->lambda, topk_idx, topk_w, s),
                          "gate and router launch");
    if (Wg) {
        CHECK(hip_status(moe_launch_gate(p->dtype, x, Wg, bg, logits, p->T, p->d, p->E, s), "gate launch"));
    }
    return hip_status(moe_launch_router(logits, p->T, p->E, p->k, p->normalize, p->lambda, topk_idx, topk_w, s),
                      "router launch");
}

moe_status do_permute(const moe_problem* p, const int32_t* topk_idx, const void* x, int32_t* counts,
                      int32_t* offsets, int32_t* slot, int32_t* src_token, void* x_perm /* nullable */, void* ws,
                      hipStream_t s)
{
    const Layout L = layout_of(p);
    return hip_status(moe_launch_permute(p->dtype, topk_idx, x, p->T, p->d, p->E, p->k, capacity_of(p), counts,
                                         offsets, slot, src_token, x_perm, at<int32_t>(ws, L.chunk_cnt), s),
                      "permute launch");
}

// Expected rows per expert: T*k/E, or the capacity when that is smaller.
int mean_rows_of(const moe_problem* p)
{
    long long m = (long long)p->T * p->k / p->E;
    const long long C = capacity_of(p);
    if (C >= 0 && C < m)
        m = C;
    return (int)std::min<long long>(m, INT32_MAX);
}

// partial: the tail-split workspace (nullable: no split).  gather
// (nullable): A is x itself and permuted row r reads row gather[r] of x.
moe_status do_up(const moe_problem* p, const void* A, const int32_t* gather, const int32_t* offsets, const void* W1,
                 void* h, float* partial, hipStream_t s, void* u_out = nullptr)
{
    const int epi = p->act == MOE_ACT_SWIGLU ? 2 : 1;
    return hip_status(moe_launch_grouped_gemm(p->dtype, epi, A, gather, p->T, W1, h, offsets, p->E, p->d, n1_of(p),
                                              p->F, p->F, p->T * p->k, mean_rows_of(p), cu_count(), partial, nullptr,
                                              u_out, n1_of(p), s),
                      "expert up launch");
}

moe_status do_down(const moe_problem* p, const void* h, const int32_t* offsets, const void* W2, void* y_perm,
                   float* partial, hipStream_t s)
{
    return hip_status(moe_launch_grouped_gemm(p->dtype, 0, h, nullptr, 0, W2, y_perm, offsets, p->E, p->F, p->d,
                                              p->d, p->F, p->T * p->k, mean_rows_of(p), cu_count(), partial, nullptr,
                                              nullptr, 0, s),
                      "expert down launch");
}

moe_status do_combine(const moe_problem* p, const void* y_perm, const int32_t* slot, const float* topk_w,
                      const void* y_add, void* y, hipStream_t s)
{
    return hip_status(moe_launch_combine(p->dtype, y_perm, slot, topk_w, y_add, p->T, p->d, p->k, p->T * p->k, y, s),
                      "combine launch");
}

// ---- shared expert: a dense expert FFN over all T rows (E = 1, no offsets)
moe_status check_shared(const moe_problem* p, int32_t Fs)
{
    CHECK(check_problem(p));
    if (Fs < 64 || Fs > kMaxDim || Fs % 64)
        return fail(MOE_ERR_UNSUPPORTED, "Fs=%d must be a multiple of 64 in [64, %d]", Fs, kMaxDim);
    const long long n1s = p->act == MOE_ACT_SWIGLU ? 2LL * Fs : Fs;
    if ((long long)p->T * std::max<long long>(n1s, p->d) >= (1LL << 40))
        return fail(MOE_ERR_UNSUPPORTED, "problem too large");
    if (n1s * p->d * (long long)elem_bytes(p) >= (1LL << 31) ||
        (long long)p->d * Fs * (long long)elem_bytes(p) >= (1LL << 31))
        return fail(MOE_ERR_UNSUPPORTED, "the shared expert's weights must stay below 2 GiB");
    return MOE_OK;
}

struct SharedLayout {
    size_t h, partial, total;
};

SharedLayout shared_layout_of(const moe_problem* p, int32_t Fs)
{
    SharedLayout L;
    L.h = 0;
    L.partial = round_up((size_t)p->T * Fs * elem_bytes(p));
    L.total = L.partial + round_up(moe_grouped_gemm_partial_bytes(p->dtype, p->T));
    return L;
}

// ---- FP8 experts: E4M3 weights and activations with power-of-two row scales
moe_status check_fp8(const moe_problem* p)
{
    CHECK(check_problem(p));
    if (p->dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "the FP8 path takes bf16 activations (dtype MOE_BF16)");
    if (p->d % 128 || p->F % 128)
        return fail(MOE_ERR_UNSUPPORTED, "the FP8 path needs d and F multiples of 128 (d=%d, F=%d)", p->d, p->F);
    return MOE_OK;
}

// Whether the FP8 codes of x (one byte per value) can be read through
// src_token: the gather addresses them with 32-bit byte offsets, like x in
// the bf16 path.
bool gather_ok_fp8(const moe_problem* p)
{
    return (unsigned long long)p->T * p->d < kGatherBytes;
}

// The bf16 layout, then the codes and scales of x and h.
struct LayoutFp8 {
    Layout base;
    size_t xq, xs, hq, hs, total;
};

LayoutFp8 layout_fp8_of(const moe_problem* p)
{
    LayoutFp8 L;
    L.base = layout_of(p);
    const size_t T = (size_t)p->T, k = (size_t)p->k;
    size_t off = L.base.total;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += round_up(bytes);
        return at;
    };
    L.xq = take(T * p->d);
    L.xs = take(T * 4);
    L.hq = take(T * k * p->F);
    L.hs = take(T * k * 4);
    L.total = off;
    return L;
}

moe_status check_ws_fp8(const moe_problem* p, const void* ws, size_t ws_bytes)
{
    const size_t need = layout_fp8_of(p).total;
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, need);
    return check_ptr(ws, "ws", 16);
}

moe_status do_up_fp8(const moe_problem* p, const void* xq, const float* xs, const int32_t* gather,
                     const int32_t* offsets, const void* W1q, const float* w1s, void* h, float* partial,
                     hipStream_t s)
{
    const int epi = p->act == MOE_ACT_SWIGLU ? 2 : 1;
    return hip_status(moe_launch_grouped_gemm_fp8(epi, xq, gather, p->T, W1q, h, offsets, p->E, p->d, n1_of(p), p->F,
                                                  p->F, p->T * p->k, mean_rows_of(p), cu_count(), partial, xs, w1s,
                                                  s),
                      "FP8 expert up launch");
}

moe_status do_down_fp8(const moe_problem* p, const void* hq, const float* hs, const int32_t* offsets,
                       const void* W2q, const float* w2s, void* y_perm, float* partial, hipStream_t s)
{
    return hip_status(moe_launch_grouped_gemm_fp8(0, hq, nullptr, 0, W2q, y_perm, offsets, p->E, p->F, p->d, p->d,
                                                  p->F, p->T * p->k, mean_rows_of(p), cu_count(), partial, hs, w2s,
                                                  s),
                      "FP8 expert down launch");
}

// ---- backward
constexpr int kSegAlign = 64;  // padded expert segments of the weight-gradient GEMMs' K

struct LayoutBwd {
    size_t d_yp, d_w, dz, du, dx_perm, W1T, W2T, kofs, d_ypT, hT, duT, xpT, gate, partial, total;
    int ld;
};

LayoutBwd layout_bwd_of(const moe_problem* p)
{
    LayoutBwd L;
    const size_t T = (size_t)p->T, k = (size_t)p->k, E = (size_t)p->E, d = (size_t)p->d, F = (size_t)p->F;
    const size_t n1 = (size_t)n1_of(p), b = elem_bytes(p);
    L.ld = (int)(((T * k + kSegAlign * E) + 63) / 64 * 64);
    const size_t ld = (size_t)L.ld;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += round_up(bytes);
        return at;
    };
    L.d_yp = take(T * k * d * b);
    L.d_w = take(T * k * 4);
    L.dz = take(T * E * 4);
    L.du = take(T * k * n1 * b);
    L.dx_perm = take(T * k * d * b);
    // transposed weights: fp32 only (the bf16 GEMMs read W1 and W2 transposed in place)
    const bool wt = p->dtype == MOE_BF16;
    L.W1T = take(wt ? 0 : E * n1 * d * b);
    L.W2T = take(wt ? 0 : E * d * F * b);
    L.kofs = take((E + 1) * 4);
    L.d_ypT = take(d * ld * b);
    L.hT = take(F * ld * b);
    L.duT = take(n1 * ld * b);
    L.xpT = take(d * ld * b);
    L.gate = take(moe_gate_wgrad_partial_bytes(p->T, p->d, p->E));
    L.partial = take(moe_grouped_gemm_partial_bytes(p->dtype, mean_rows_of(p)));
    L.total = off;
    return L;
}

moe_status check_bwd(const moe_problem* p)
{
    CHECK(check_problem(p));
    // the weight-gradient GEMMs address [rows][ld] operands with 32-bit offsets
    const LayoutBwd L = layout_bwd_of(p);
    const long long widest = std::max<long long>(std::max(p->d, p->F), n1_of(p));
    if (widest * L.ld * (long long)elem_bytes(p) >= 0xF0000000LL)
        return fail(MOE_ERR_UNSUPPORTED, "the backward's transposed operands exceed 32-bit offsets");
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s)
{
    switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

moe_status moe_capacity(const moe_problem* p, int32_t* C)
{
    CHECK(check_problem(p));
    if (!C)
        return fail(MOE_ERR_INVALID_ARG, "C is NULL");
    const long long c = capacity_of(p);
    *C = c > (long long)INT32_MAX ? INT32_MAX : (int32_t)c;
    return ok();
}

moe_status moe_workspace_size(const moe_problem* p, size_t* bytes)
{
    CHECK(check_problem(p));
    if (!bytes)
        return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = layout_of(p).total;
    return ok();
}

moe_status moe_route(const moe_problem* p, const void* x, const void* Wg, const float* bg, float* logits,
                     int32_t* topk_idx, float* topk_w, void* stream)
{
    CHECK(check_problem(p));
    if ((x == nullptr) != (Wg == nullptr))
        return fail(MOE_ERR_INVALID_ARG, "x and Wg must both be given (gate) or both be NULL (logits given)");
    if (p->T == 0)
        return ok();
    if (Wg) {
        CHECK(check_ptr(x, "x", 16));
        CHECK(check_ptr(Wg, "Wg", 16));
        if (bg)
            CHECK(check_ptr(bg, "bg", 4));
    }
    CHECK(check_ptr(logits, "logits", 4));
    CHECK(check_ptr(topk_idx, "topk_idx", 4));
    CHECK(check_ptr(topk_w, "topk_w", 4));
    CHECK(do_route(p, x, Wg, bg, logits, topk_idx, topk_w, (hipStream_t)stream));
    return ok();
}

moe_status moe_permute(const moe_problem* p, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* slot, int32_t* src_token, void* x_perm, void* ws, size_t ws_bytes,
                       void* stream)
{
    CHECK(check_problem(p));
    if (p->T == 0)
        return ok();
    CHECK(check_ptr(topk_idx, "topk_idx", 4));
    if (x_perm) {
        CHECK(check_ptr(x, "x", 16));
        CHECK(check_ptr(x_perm, "x_perm", 16));
    }
    CHECK(check_ptr(counts, "counts", 4));
    CHECK(check_ptr(offsets, "offsets", 4));
    CHECK(check_ptr(slot, "slot", 4));
    CHECK(check_ptr(src_token, "src_token", 4));
    CHECK(check_ws(p, ws, ws_bytes));
    CHECK(do_permute(p, topk_idx, x, counts, offsets, slot, src_token, x_perm, ws, (hipStream_t)stream));
    return ok();
}

moe_status moe_expert_up(const moe_problem* p, const void* a, const int32_t* src_token, const int32_t* offsets,
                         const void* W1, void* h, void* ws, size_t ws_bytes, void* stream)
{
    CHECK(check_problem(p));
    if (p->T == 0)
        return ok();
    CHECK(check_ptr(a, src_token ? "x" : "x_perm", 16));
    if (src_token) {
        CHECK(check_ptr(src_token, "src_token", 4));
        if (!gather_ok(p))
            return fail(MOE_ERR_UNSUPPORTED, "x of %llu bytes is too large to gather; pass x_perm",
                        (unsigned long long)p->T * p->d * elem_bytes(p));
    }
    CHECK(check_ptr(offsets, "offsets", 4));
    CHECK(check_ptr(W1, "W1", 16));
    CHECK(check_ptr(h, "h", 16));
    if (ws)
        CHECK(check_ws(p, ws, ws_bytes));
    float* partial = ws ? at<float>(ws, layout_of(p).partial) : nullptr;
    CHECK(do_up(p, a, src_token, offsets, W1, h, partial, (hipStream_t)stream));
    return ok();
}

moe_status moe_expert_down(const moe_problem* p, const void* h, const int32_t* offsets, const void* W2,
                           void* y_perm, void* ws, size_t ws_bytes, void* stream)
{
    CHECK(check_problem(p));
    if (p->T == 0)
        return ok();
    CHECK(check_ptr(h, "h", 16));
    CHECK(check_ptr(offsets, "offsets", 4));
    CHECK(check_ptr(W2, "W2", 16));
    CHECK(check_ptr(y_perm, "y_perm", 16));
    if (ws)
        CHECK(check_ws(p, ws, ws_bytes));
    float* partial = ws ? at<float>(ws, layout_of(p).partial) : nullptr;
    CHECK(do_down(p, h, offsets, W2, y_perm, partial, (hipStream_t)stream));
    return ok();
}

moe_status moe_grouped_ffn(const moe_problem* p, const void* x_perm, const int32_t* offsets, const void* W1,
                           const void* W2, void* y_perm, void* ws, size_t ws_bytes, void* stream)
{
    CHECK(check_problem(p));
    if (p->T == 0)
        return ok();
    CHECK(check_ptr(x_perm, "x_perm", 16));
    CHECK(check_ptr(offsets, "offsets", 4));
    CHECK(check_ptr(W1, "W1", 16));
    CHECK(check_ptr(W2, "W2", 16));
    CHECK(check_ptr(y_perm, "y_perm", 16));
    CHECK(check_ws(p, ws, ws_bytes));
    const Layout L = layout_of(p);
    void* h = at<char>(ws, L.h);
    float* partial = at<float>(ws, L.partial);
    CHECK(do_up(p, x_perm, nullptr, offsets, W1, h, partial, (hipStream_t)stream));
    CHECK(do_down(p, h, offsets, W2, y_perm, partial, (hipStream_t)stream));
    return ok();
}

moe_status moe_combine(const moe_problem* p, const void* y_perm, const int32_t* slot, const float* topk_w, void* y,
                       void* stream)
{
    CHECK(check_problem(p));
    if (p->T == 0)
        return ok();
    CHECK(check_ptr(y_perm, "y_perm", 16));
    CHECK(check_ptr(slot, "slot", 4));
    CHECK(check_ptr(topk_w, "topk_w", 4));
    CHECK(check_ptr(y, "y", 16));
    CHECK(do_combine(p, y_perm, slot, topk_w, nullptr, y, (hipStream_t)stream));
    return ok();
}

}  // extern "C"

namespace {

// Argument checks of moe_forward other than the workspace.
moe_status check_forward(const moe_problem* p, const void* x, const void* Wg, const float* bg, const void* W1,
                         const void* W2, const void* y, const float* logits)
{
    CHECK(check_ptr(x, "x", 16));
    CHECK(check_ptr(W1, "W1", 16));
    CHECK(check_ptr(W2, "W2", 16));
    CHECK(check_ptr(y, "y", 16));
    if (Wg) {
        CHECK(check_ptr(Wg, "Wg", 16));
        if (bg)
            CHECK(check_ptr(bg, "bg", 4));
        if (logits)
            CHECK(check_ptr(logits, "logits", 4));
    } else {
        if (!logits)
            return fail(MOE_ERR_INVALID_ARG, "logits must be given when Wg is NULL");
        CHECK(check_ptr(logits, "logits", 4));
    }
    return MOE_OK;
}

// The forward's launch sequence on a validated workspace of layout L (with
// or without the K-split partial tiles).
moe_status forward_steps(const moe_problem* p, const void* x, const void* Wg, const float* bg, const void* W1,
                         const void* W2, void* y, float* logits, const moe_route_info* info, void* ws,
                         const Layout& L, bool split, hipStream_t s)
{
    moe_route_info r = {};
    if (info)
        r = *info;
#define PICK(field, type) (r.field ? r.field : at<type>(ws, L.field))
    int32_t* topk_idx = PICK(topk_idx, int32_t);
    float* topk_w = PICK(topk_w, float);
    int32_t* counts = PICK(counts, int32_t);
    int32_t* offsets = PICK(offsets, int32_t);
    int32_t* slot = PICK(slot, int32_t);
    int32_t* src_token = PICK(src_token, int32_t);
#undef PICK
    const void* ptrs[] = {topk_idx, topk_w, counts, offsets, slot, src_token};
    for (const void* q : ptrs)
        CHECK(check_ptr(q, "route info field", 4));
    float* z = logits ? logits : at<float>(ws, L.logits);
    float* partial = split ? at<float>(ws, L.partial) : nullptr;
    void* h = at<char>(ws, L.h);
    void* y_perm = at<char>(ws, L.y_perm);
    CHECK(do_route(p, Wg ? x : nullptr, Wg, bg, z, topk_idx, topk_w, s));
    // the up projection reads the token rows of x through src_token, so the
    // permutation writes no x_perm copy (unless x is beyond 32-bit offsets)
    if (gather_ok(p)) {
        CHECK(do_permute(p, topk_idx, x, counts, offsets, slot, src_token, nullptr, ws, s));
        CHECK(do_up(p, x, src_token, offsets, W1, h, partial, s));
    } else {
        void* x_perm = at<char>(ws, L.x_perm);
        CHECK(do_permute(p, topk_idx, x, counts, offsets, slot, src_token, x_perm, ws, s));
        CHECK(do_up(p, x_perm, nullptr, offsets, W1, h, partial, s));
    }
    CHECK(do_down(p, h, offsets, W2, y_perm, partial, s));
    CHECK(do_combine(p, y_perm, slot, topk_w, nullptr, y, s));
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_problem* p, const void* x, const void* Wg, const float* bg, const void* W1,
                       const void* W2, void* y, float* logits, const moe_route_info* info, void* ws, size_t ws_bytes,
                       void* stream)
{
    CHECK(check_problem(p));
    if (p->T == 0)
        return ok();
    CHECK(check_forward(p, x, Wg, bg, W1, W2, y, logits));
    CHECK(check_ws(p, ws, ws_bytes));
    CHECK(forward_steps(p, x, Wg, bg, W1, W2, y, logits, info, ws, layout_of(p), true, (hipStream_t)stream));
    return ok();
}

moe_status moe_forward_noalloc(const moe_problem* p, const void* x, const void* Wg, const float* bg, const void* W1,
                               const void* W2, void* y, float* logits, const moe_route_info* info, void* stream)
{
    CHECK(check_problem(p));
    if (p->T == 0)
        return ok();
    CHECK(check_forward(p, x, Wg, bg, W1, W2, y, logits));
    const Layout L = layout_of(p, false);
    if (L.total > kScratchBytes)
        return fail(MOE_ERR_WORKSPACE, "the problem needs %zu bytes of scratch; the allocation-free forward has %zu",
                    L.total, kScratchBytes);
    void* ws = nullptr;
    CHECK(scratch_address(&ws));
    CHECK(forward_steps(p, x, Wg, bg, W1, W2, y, logits, info, ws, L, false, (hipStream_t)stream));
    return ok();
}

moe_status moe_router_stats(const moe_problem* p, const float* logits, const int32_t* counts,
                            const int32_t* offsets, float* frac, float* mean_prob, float* scalars, void* ws,
                            size_t ws_bytes, void* stream)
{
    CHECK(check_problem(p));
    if (p->T == 0)
        return ok();
    CHECK(check_ptr(logits, "logits", 4));
    CHECK(check_ptr(counts, "counts", 4));
    CHECK(check_ptr(offsets, "offsets", 4));
    CHECK(check_ptr(frac, "frac", 4));
    CHECK(check_ptr(mean_prob, "mean_prob", 4));
    CHECK(check_ptr(scalars, "scalars", 4));
    CHECK(check_ws(p, ws, ws_bytes));
    double* partial = at<double>(ws, layout_of(p).stats);
    CHECK(hip_status(moe_launch_router_stats(logits, p->T, p->E, p->k, p->normalize, p->lambda, counts, offsets,
                                             partial, frac, mean_prob, scalars, (hipStream_t)stream),
                     "router statistics launch"));
    return ok();
}

moe_status moe_shared_workspace_size(const moe_problem* p, int32_t Fs, size_t* bytes)
{
    CHECK(check_shared(p, Fs));
    if (!bytes)
        return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = shared_layout_of(p, Fs).total;
    return ok();
}

moe_status moe_shared_expert(const moe_problem* p, int32_t Fs, const void* x, const void* Ws1, const void* Ws2,
                             void* y_shared, void* ws, size_t ws_bytes, void* stream)
{
    CHECK(check_shared(p, Fs));
    if (p->T == 0)
        return ok();
    CHECK(check_ptr(x, "x", 16));
    CHECK(check_ptr(Ws1, "Ws1", 16));
    CHECK(check_ptr(Ws2, "Ws2", 16));
    CHECK(check_ptr(y_shared, "y_shared", 16));
    const SharedLayout L = shared_layout_of(p, Fs);
    if (ws_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, L.total);
    CHECK(check_ptr(ws, "ws", 16));
    void* h = at<char>(ws, L.h);
    float* partial = at<float>(ws, L.partial);
    const int epi = p->act == MOE_ACT_SWIGLU ? 2 : 1;
    const int n1s = p->act == MOE_ACT_SWIGLU ? 2 * Fs : Fs;
    hipStream_t s = (hipStream_t)stream;
    CHECK(hip_status(moe_launch_grouped_gemm(p->dtype, epi, x, nullptr, 0, Ws1, h, nullptr, 1, p->d, n1s, Fs, Fs,
                                             p->T, p->T, cu_count(), partial, nullptr, nullptr, 0, s),
                     "shared expert up launch"));
    CHECK(hip_status(moe_launch_grouped_gemm(p->dtype, 0, h, nullptr, 0, Ws2, y_shared, nullptr, 1, Fs, p->d, p->d,
                                             Fs, p->T, p->T, cu_count(), partial, nullptr, nullptr, 0, s),
                     "shared expert down launch"));
    return ok();
}

moe_status moe_combine_shared(const moe_problem* p, const void* y_perm, const int32_t* slot, const float* topk_w,
                              const void* y_shared, void* y, void* stream)
{
    CHECK(check_problem(p));
    if (p->T == 0)
        return ok();
    CHECK(check_ptr(y_perm, "y_perm", 16));
    CHECK(check_ptr(slot, "slot", 4));
    CHECK(check_ptr(topk_w, "topk_w", 4));
    CHECK(check_ptr(y_shared, "y_shared", 16));
    CHECK(check_ptr(y, "y", 16));
    CHECK(do_combine(p, y_perm, slot, topk_w, y_shared, y, (hipStream_t)stream));
    return ok();
}

moe_status moe_fp8_workspace_size(const moe_problem* p, size_t* bytes)
{
    CHECK(check_fp8(p));
    if (!bytes)
        return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = layout_fp8_of(p).total;
    return ok();
}

moe_status moe_quantize_fp8(const void* src, int32_t src_dtype, int64_t rows, int32_t K, uint8_t* codes,
                            float* scales, void* stream)
{
    if (src_dtype != MOE_F32 && src_dtype != MOE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "src_dtype=%d is neither MOE_F32 nor MOE_BF16", src_dtype);
    if (rows < 0)
        return fail(MOE_ERR_INVALID_ARG, "rows=%lld is negative", (long long)rows);
    if (K < 64 || K > kMaxDim || K % 64)
        return fail(MOE_ERR_UNSUPPORTED, "K=%d must be a multiple of 64 in [64, %d]", K, kMaxDim);
    if (rows > ((long long)1 << 40) / K || rows > INT32_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "too many rows");
    if (rows == 0)
        return ok();
    CHECK(check_ptr(src, "src", 16));
    CHECK(check_ptr(codes, "codes", 8));
    CHECK(check_ptr(scales, "scales", 4));
    CHECK(hip_status(moe_launch_quantize_fp8(src_dtype == MOE_F32 ? 0 : 1, src, rows, K, codes, scales,
                                             (hipStream_t)stream),
                     "FP8 quantisation launch"));
    return ok();
}

moe_status moe_expert_up_fp8(const moe_problem* p, const uint8_t* aq, const float* as, const int32_t* src_token,
                             const int32_t* offsets, const uint8_t* W1q, const float* w1s, void* h, void* ws,
                             size_t ws_bytes, void* stream)
{
    CHECK(check_fp8(p));
    if (p->T == 0)
        return ok();
    CHECK(check_ptr(aq, src_token ? "xq" : "x_perm codes", 16));
    CHECK(check_ptr(as, "activation scales", 4));
    if (src_token) {
        CHECK(check_ptr(src_token, "src_token", 4));
        if (!gather_ok_fp8(p))
            return fail(MOE_ERR_UNSUPPORTED, "x codes of %llu bytes are too large to gather; pass permuted codes",
                        (unsigned long long)p->T * p->d);
    }
    CHECK(check_ptr(offsets, "offsets", 4));
    CHECK(check_ptr(W1q, "W1q", 16));
    CHECK(check_ptr(w1s, "w1s", 4));
    CHECK(check_ptr(h, "h", 16));
    if (ws)
        CHECK(check_ws(p, ws, ws_bytes));
    float* partial = ws ? at<float>(ws, layout_of(p).partial) : nullptr;
    CHECK(do_up_fp8(p, aq, as, src_token, offsets, W1q, w1s, h, partial, (hipStream_t)stream));
    return ok();
}

moe_status moe_expert_down_fp8(const moe_problem* p, const uint8_t* hq, const float* hs, const int32_t* offsets,
                               const uint8_t* W2q, const float* w2s, void* y_perm, void* ws, size_t ws_bytes,
                               void* stream)
{
    CHECK(check_fp8(p));
    if (p->T == 0)
        return ok();
    CHECK(check_ptr(hq, "hq", 16));
    CHECK(check_ptr(hs, "hs", 4));
    CHECK(check_ptr(offsets, "offsets", 4));
    CHECK(check_ptr(W2q, "W2q", 16));
    CHECK(check_ptr(w2s, "w2s", 4));
    CHECK(check_ptr(y_perm, "y_perm", 16));
    if (ws)
        CHECK(check_ws(p, ws, ws_bytes));
    float* partial = ws ? at<float>(ws, layout_of(p).partial) : nullptr;
    CHECK(do_down_fp8(p, hq, hs, offsets, W2q, w2s, y_perm, partial, (hipStream_t)stream));
    return ok();
}

moe_status moe_forward_fp8(const moe_problem* p, const void* x, const void* Wg, const float* bg, const uint8_t* W1q,
                           const float* w1s, const uint8_t* W2q, const float* w2s, void* y, float* logits,
                           const moe_route_info* info, void* ws, size_t ws_bytes, void* stream)
{
    CHECK(check_fp8(p));
    if (p->T == 0)
        return ok();
    if (!gather_ok_fp8(p))
        return fail(MOE_ERR_UNSUPPORTED, "x codes of %llu bytes are too large to gather (limit 0xF0000000 bytes)",
                    (unsigned long long)p->T * p->d);
    CHECK(check_ptr(x, "x", 16));
    CHECK(check_ptr(W1q, "W1q", 16));
    CHECK(check_ptr(w1s, "w1s", 4));
    CHECK(check_ptr(W2q, "W2q", 16));
    CHECK(check_ptr(w2s, "w2s", 4));
    CHECK(check_ptr(y, "y", 16));
    if (Wg) {
        CHECK(check_ptr(Wg, "Wg", 16));
        if (bg)
            CHECK(check_ptr(bg, "bg", 4));
        if (logits)
            CHECK(check_ptr(logits, "logits", 4));
    } else {
        if (!logits)
            return fail(MOE_ERR_INVALID_ARG, "logits must be given when Wg is NULL");
        CHECK(check_ptr(logits, "logits", 4));
    }
    CHECK(check_ws_fp8(p, ws, ws_bytes));
    const LayoutFp8 LF = layout_fp8_of(p);
    const Layout& L = LF.base;
    moe_route_info r = {};
    if (info)
        r = *info;
#define PICK(field, type) (r.field ? r.field : at<type>(ws, L.field))
    int32_t* topk_idx = PICK(topk_idx, int32_t);
    float* topk_w = PICK(topk_w, float);
    int32_t* counts = PICK(counts, int32_t);
    int32_t* offsets = PICK(offsets, int32_t);
    int32_t* slot = PICK(slot, int32_t);
    int32_t* src_token = PICK(src_token, int32_t);
#undef PICK
    const void* ptrs[] = {topk_idx, topk_w, counts, offsets, slot, src_token};
    for (const void* q : ptrs)
        CHECK(check_ptr(q, "route info field", 4));
    float* z = logits ? logits : at<float>(ws, L.logits);
    float* partial = at<float>(ws, L.partial);
    void* h = at<char>(ws, L.h);
    void* y_perm = at<char>(ws, L.y_perm);
    uint8_t* xq = at<uint8_t>(ws, LF.xq);
    float* xs = at<float>(ws, LF.xs);
    uint8_t* hq = at<uint8_t>(ws, LF.hq);
    float* hs = at<float>(ws, LF.hs);
    hipStream_t s = (hipStream_t)stream;
    CHECK(do_route(p, Wg ? x : nullptr, Wg, bg, z, topk_idx, topk_w, s));
    CHECK(do_permute(p, topk_idx, x, counts, offsets, slot, src_token, nullptr, ws, s));
    CHECK(hip_status(moe_launch_quantize_fp8(1, x, p->T, p->d, xq, xs, s), "FP8 quantisation launch"));
    CHECK(do_up_fp8(p, xq, xs, src_token, offsets, W1q, w1s, h, partial, s));
    // h rows past offsets[E] are not written by the GEMM; quantising all T*k
    // rows keeps the launch free of a host read of offsets (those codes are
    // never used)
    CHECK(hip_status(moe_launch_quantize_fp8(1, h, (long long)p->T * p->k, p->F, hq, hs, s),
                     "FP8 quantisation launch"));
    CHECK(do_down_fp8(p, hq, hs, offsets, W2q, w2s, y_perm, partial, s));
    CHECK(do_combine(p, y_perm, slot, topk_w, nullptr, y, s));
    return ok();
}

moe_status moe_forward_train(const moe_problem* p, const void* x, const void* Wg, const float* bg, const void* W1,
                             const void* W2, void* y, float* logits, const moe_route_info* info,
                             const moe_saved* saved, void* ws, size_t ws_bytes, void* stream)
{
    CHECK(check_problem(p));
    if (p->T == 0)
        return ok();
    if (!info || !saved)
        return fail(MOE_ERR_INVALID_ARG, "info and saved are required");
    CHECK(check_ptr(x, "x", 16));
    CHECK(check_ptr(W1, "W1", 16));
    CHECK(check_ptr(W2, "W2", 16));
    CHECK(check_ptr(y, "y", 16));
    CHECK(check_ptr(logits, "logits", 4));
    if (Wg) {
        CHECK(check_ptr(Wg, "Wg", 16));
        if (bg)
            CHECK(check_ptr(bg, "bg", 4));
    }
    const void* rp[] = {info->topk_idx, info->topk_w, info->counts, info->offsets, info->slot, info->src_token};
    for (const void* q : rp)
        CHECK(check_ptr(q, "route info field", 4));
    CHECK(check_ptr(saved->u, "saved u", 16));
    CHECK(check_ptr(saved->h, "saved h", 16));
    CHECK(check_ptr(saved->y_perm, "saved y_perm", 16));
    CHECK(check_ws(p, ws, ws_bytes));
    const Layout L = layout_of(p);
    float* partial = at<float>(ws, L.partial);
    hipStream_t s = (hipStream_t)stream;
    CHECK(do_route(p, Wg ? x : nullptr, Wg, bg, logits, info->topk_idx, info->topk_w, s));
    if (gather_ok(p)) {
        CHECK(do_permute(p, info->topk_idx, x, info->counts, info->offsets, info->slot, info->src_token, nullptr, ws,
                         s));
        CHECK(do_up(p, x, info->src_token, info->offsets, W1, saved->h, partial, s, saved->u));
    } else {
        void* x_perm = at<char>(ws, L.x_perm);
        CHECK(do_permute(p, info->topk_idx, x, info->counts, info->offsets, info->slot, info->src_token, x_perm, ws,
                         s));
        CHECK(do_up(p, x_perm, nullptr, info->offsets, W1, saved->h, partial, s, saved->u));
    }
    CHECK(do_down(p, saved->h, info->offsets, W2, saved->y_perm, partial, s));
    CHECK(do_combine(p, saved->y_perm, info->slot, info->topk_w, nullptr, y, s));
    return ok();
}

moe_status moe_backward_workspace_size(const moe_problem* p, size_t* bytes)
{
    CHECK(check_bwd(p));
    if (!bytes)
        return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = layout_bwd_of(p).total;
    return ok();
}

moe_status moe_backward(const moe_problem* p, const void* dy, const void* x, const void* Wg, const void* W1,
                        const void* W2, const float* logits, const moe_route_info* info, const moe_saved* saved,
                        const moe_router_losses* losses, void* dx, float* dWg, float* dbg, float* dW1, float* dW2,
                        void* ws, size_t ws_bytes, void* stream)
{
    CHECK(check_bwd(p));
    hipStream_t s = (hipStream_t)stream;
    const int T = p->T, d = p->d, E = p->E, k = p->k, F = p->F, n1 = n1_of(p), rows = T * k;
    if (T == 0) {  // no tokens: every weight gradient is zero
        CHECK(check_ptr(dW1, "dW1", 16));
        CHECK(check_ptr(dW2, "dW2", 16));
        CHECK(hip_status(moe_launch_zero(dW1, (size_t)E * n1 * d, s), "zero fill launch"));
        CHECK(hip_status(moe_launch_zero(dW2, (size_t)E * d * F, s), "zero fill launch"));
        if (Wg) {
            CHECK(check_ptr(dWg, "dWg", 4));
            CHECK(check_ptr(dbg, "dbg", 4));
            CHECK(hip_status(moe_launch_zero(dWg, (size_t)E * d, s), "zero fill launch"));
            CHECK(hip_status(moe_launch_zero(dbg, (size_t)E, s), "zero fill launch"));
        }
        return ok();
    }
    if (!info || !saved)
        return fail(MOE_ERR_INVALID_ARG, "info and saved are required");
    CHECK(check_ptr(dy, "dy", 16));
    CHECK(check_ptr(x, "x", 16));
    CHECK(check_ptr(W1, "W1", 16));
    CHECK(check_ptr(W2, "W2", 16));
    CHECK(check_ptr(logits, "logits", 4));
    const void* rp[] = {info->topk_idx, info->topk_w, info->offsets, info->slot, info->src_token};
    for (const void* q : rp)
        CHECK(check_ptr(q, "route info field", 4));
    CHECK(check_ptr(saved->u, "saved u", 16));
    CHECK(check_ptr(saved->h, "saved h", 16));
    CHECK(check_ptr(saved->y_perm, "saved y_perm", 16));
    const float aux_coef = losses ? losses->aux_coef : 0.0f, z_coef = losses ? losses->z_coef : 0.0f;
    if (!std::isfinite(aux_coef) || !std::isfinite(z_coef))
        return fail(MOE_ERR_INVALID_ARG, "balancing-loss coefficients must be finite");
    if (aux_coef != 0.0f)
        CHECK(check_ptr(info->counts, "info counts", 4));
    CHECK(check_ptr(dx, "dx", 16));
    CHECK(check_ptr(dW1, "dW1", 16));
    CHECK(check_ptr(dW2, "dW2", 16));
    if (Wg) {
        CHECK(check_ptr(Wg, "Wg", 16));
        CHECK(check_ptr(dWg, "dWg", 4));
        CHECK(check_ptr(dbg, "dbg", 4));
    }
    const LayoutBwd L = layout_bwd_of(p);
    if (ws_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, L.total);
    CHECK(check_ptr(ws, "ws", 16));
    const int dt = p->dtype == MOE_F32 ? 0 : 1;
    void* d_yp = at<char>(ws, L.d_yp);
    float* d_w = at<float>(ws, L.d_w);
    float* dz = at<float>(ws, L.dz);
    void* du = at<char>(ws, L.du);
    void* dx_perm = at<char>(ws, L.dx_perm);
    void* W1T = at<char>(ws, L.W1T);
    void* W2T = at<char>(ws, L.W2T);
    int32_t* kofs = at<int32_t>(ws, L.kofs);
    float* partial = at<float>(ws, L.partial);
    const int32_t* offsets = info->offsets;
    // combine and router
    CHECK(hip_status(moe_launch_combine_bwd(dt, dy, saved->y_perm, info->slot, info->topk_w, T, d, k, rows, d_yp, d_w,
                                            s), "combine backward launch"));
    if (Wg)  // with given logits nothing reads the logit gradient
        CHECK(hip_status(moe_launch_router_bwd(logits, info->topk_idx, info->slot, d_w, T, E, k, p->normalize,
                                               p->lambda, aux_coef, z_coef, info->counts, dz, s),
                         "router backward launch"));
    // input gradients of the expert layers: dh = d_yp W2[e] (+ activation backward), dx_perm = du W1[e]
    const int depi = p->act == MOE_ACT_SWIGLU ? 4 : 3;
    if (p->dtype == MOE_BF16) {
        // W2[e] is [d][F] and W1[e] is [n1][d]: K-major weight operands, read as stored
        CHECK(hip_status(moe_launch_grouped_gemm_wt(depi, d_yp, W2, du, offsets, E, d, F, n1, F, rows,
                                                    mean_rows_of(p), cu_count(), partial, saved->u, n1, s),
                         "expert down backward launch"));
        CHECK(hip_status(moe_launch_grouped_gemm_wt(0, du, W1, dx_perm, offsets, E, n1, d, d, d, rows,
                                                    mean_rows_of(p), cu_count(), partial, nullptr, 0, s),
                         "expert up backward launch"));
    } else {
        CHECK(hip_status(moe_launch_transpose(dt, W2, E, d, F, W2T, s), "transpose launch"));
        CHECK(hip_status(moe_launch_transpose(dt, W1, E, n1, d, W1T, s), "transpose launch"));
        CHECK(hip_status(moe_launch_grouped_gemm(p->dtype, depi, d_yp, nullptr, 0, W2T, du, offsets, E, d, F, n1, F,
                                                 rows, mean_rows_of(p), cu_count(), partial, saved->u, nullptr, n1, s),
                         "expert down backward launch"));
        CHECK(hip_status(moe_launch_grouped_gemm(p->dtype, 0, du, nullptr, 0, W1T, dx_perm, offsets, E, n1, d, d, d,
                                                 rows, mean_rows_of(p), cu_count(), partial, nullptr, nullptr, 0, s),
                         "expert up backward launch"));
    }
    // weight gradients: per expert, reductions over its rows
    CHECK(hip_status(moe_launch_kofs(offsets, E, rows, kSegAlign, kofs, s), "segment offsets launch"));
    void* d_ypT = at<char>(ws, L.d_ypT);
    void* hT = at<char>(ws, L.hT);
    void* duT = at<char>(ws, L.duT);
    void* xpT = at<char>(ws, L.xpT);
    CHECK(hip_status(moe_launch_seg_transpose(dt, d_yp, nullptr, 0, offsets, kofs, E, rows, d, L.ld, d_ypT, s),
                     "segment transpose launch"));
    CHECK(hip_status(moe_launch_seg_transpose(dt, saved->h, nullptr, 0, offsets, kofs, E, rows, F, L.ld, hT, s),
                     "segment transpose launch"));
    CHECK(hip_status(moe_launch_seg_transpose(dt, du, nullptr, 0, offsets, kofs, E, rows, n1, L.ld, duT, s),
                     "segment transpose launch"));
    CHECK(hip_status(moe_launch_seg_transpose(dt, x, info->src_token, T, offsets, kofs, E, rows, d, L.ld, xpT, s),
                     "segment transpose launch"));
    CHECK(hip_status(moe_launch_grouped_gemm_kgrp(dt, d_ypT, hT, dW2, kofs, E, L.ld, d, F, cu_count(), s),
                     "weight gradient launch"));
    CHECK(hip_status(moe_launch_grouped_gemm_kgrp(dt, duT, xpT, dW1, kofs, E, L.ld, n1, d, cu_count(), s),
                     "weight gradient launch"));
    // input gradient, and the gate's
    CHECK(hip_status(moe_launch_unpermute_bwd(dt, dx_perm, info->slot, T, d, k, rows, dz, Wg, E, dx, s),
                     "un-permute backward launch"));
    if (Wg)
        CHECK(hip_status(moe_launch_gate_wgrad(dt, dz, x, T, d, E, at<float>(ws, L.gate), dWg, dbg, s),
                         "gate gradient launch"));
    return ok();
}

}  // extern "C"
