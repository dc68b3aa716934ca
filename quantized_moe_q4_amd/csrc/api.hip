// api.hip -- the library's C ABI (declared in include/moe_q4.h): argument
// validation, workspace carving and kernel launches.  Nothing here allocates,
// frees or synchronises; every launch goes on the caller's stream.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_q4.h"

namespace moeq4 {
hipError_t launch_quantize_act(const float* x, int64_t rows, int cols, bool rmsnorm, int8_t* xq, float* xd,
                               hipStream_t s);
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* wts, int32_t* offsets,
                        int32_t* sorted, hipStream_t s);
hipError_t launch_decode(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs, const uint16_t* gate_d,
                         const uint16_t* up_d, const uint16_t* down_d, int E, int H, int I, const int8_t* xq,
                         const float* xd, int T, int k, const float* topk_w, const int32_t* off,
                         const int32_t* sorted, bool accumulate, float* y, int8_t* hq, float* hd, float* o,
                         hipStream_t s);
hipError_t launch_prefill(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                          const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H, int I,
                          const int8_t* xq, const float* xd, int T, int k, const float* topk_w, const int32_t* off,
                          const int32_t* sorted, bool accumulate, float* y, int8_t* hq, float* hd, float* o,
                          hipStream_t s);
hipError_t launch_prefill_dots(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                               const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H,
                               int I, const int8_t* xq, const float* xd, int T, int k, const int32_t* off,
                               const int32_t* sorted, int which, int8_t* hq, float* hd, int32_t* dump,
                               hipStream_t s);
hipError_t launch_decode_fused(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                               const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H,
                               int I, const float* x, const float* logits, int T, int k, bool rmsnorm,
                               bool accumulate, int32_t* ids, float* wts, int32_t* offsets, int32_t* sorted,
                               float* y, int8_t* hq, float* hd, void* ctl, hipStream_t s);
bool fused_supported(int T, int k, int I);
hipError_t launch_decode_stack(const uint8_t* const* gq, const uint8_t* const* uq, const uint8_t* const* dq,
                               const uint16_t* const* gd, const uint16_t* const* ud, const uint16_t* const* dd, int L,
                               int E, int H, int I, float* h, const float* logits, int k, bool rmsnorm,
                               bool accumulate, float* h_all, int8_t* hq_all, float* hd_all, void* ws,
                               bool* too_large, hipStream_t s);
bool stack_supported(int E, int H, int I, int k);
hipError_t launch_decode_stack_batch(const uint8_t* const* gq, const uint8_t* const* uq, const uint8_t* const* dq,
                                     const uint16_t* const* gd, const uint16_t* const* ud,
                                     const uint16_t* const* dd, int L, int T, int E, int H, int I, float* h,
                                     const float* logits, int k, bool rmsnorm, bool accumulate, float* h_all,
                                     int8_t* hq_all, float* hd_all, void* ws, bool* too_large, hipStream_t s);
bool stack_batch_supported(int E, int H, int I, int T, int k);
size_t stack_batch_workspace_bytes(int L, int T, int k, int H, int I);
int stack_batch_max_layers();
size_t stack_workspace_bytes(int H);
int stack_max_layers();
hipError_t launch_prefill_a16(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                              const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H,
                              int I, const float* x, int T, int k, const float* topk_w, const int32_t* off,
                              const int32_t* sorted, bool accumulate, float* y, _Float16* x16, _Float16* h16,
                              float* o, hipStream_t s);
hipError_t launch_gemv(const uint8_t* qs, const uint16_t* d, int N, int K, const int8_t* xq, const float* xd, int T,
                       float* y, hipStream_t s);
hipError_t launch_block_dots(const uint8_t* qs, int N, int K, const int8_t* xq, int T, bool down_walk, int32_t* out,
                             hipStream_t s);
} // namespace moeq4

namespace {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_HIP; }

inline bool hidden_ok(int H) { return H == 256 || H == 512 || H == 1024 || H == 2048; }
inline bool inter_ok(int I) { return I == 256 || I == 512 || I == 1024; }

// Workspace regions (offsets documented with moe_q4_workspace_size).
// sync area of the fused decode: 4 KB of control words, then its 16 KB tagged exchange of h
constexpr size_t WS_CTL_BYTES = 4096 + 16384;

struct Ws {
    void* ctl;  // sync area of the fused decode; error word at byte 2112
    int8_t* hq; // [P][I]
    float* hd;  // [P][I/32]
    float* o;   // [P][H]: per-pair down outputs (decode's expert-major path, prefill)
};

Ws carve(void* ws, int64_t P, int H, int I)
{
    Ws w;
    w.ctl = ws;
    w.hq = (int8_t*)ws + WS_CTL_BYTES;
    w.hd = (float*)((char*)w.hq + align256((size_t)P * I));
    w.o = (float*)((char*)w.hd + align256((size_t)P * (I / 32) * sizeof(float)));
    (void)H;
    return w;
}

// Shared checks of moe_q4_decode / moe_q4_prefill arguments.
int check_layer(const moe_q4_experts* w, const int8_t* xq, const float* xd, int32_t T, int32_t k,
                const int32_t* topk_ids, const float* topk_w, const int32_t* off, const int32_t* sorted, uint32_t flags,
                const float* y, const void* ws, size_t ws_bytes, bool a16 = false)
{
    if (!w) return MOE_Q4_ERR_INVALID_ARG;
    const int E = w->num_experts, H = w->hidden, I = w->inter;
    if (E < 1 || H <= 0 || I <= 0 || H % 32 || I % 32) return MOE_Q4_ERR_INVALID_ARG;
    if (T < 0 || k < 1 || k > E) return MOE_Q4_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)MOE_Q4_ACCUMULATE) return MOE_Q4_ERR_INVALID_ARG;
    if (!w->gate_qs || !w->up_qs || !w->down_qs || !w->gate_d || !w->up_d || !w->down_d)
        return MOE_Q4_ERR_INVALID_ARG;
    const void* p16[] = {w->gate_qs, w->up_qs, w->down_qs, w->gate_d, w->up_d, w->down_d, xq};
    const void* p4[] = {xd, topk_ids, topk_w, off, sorted, y};
    if (T > 0) { // with no tokens the per-token arrays may be empty (null)
        if (!xq || !xd || !topk_ids || !topk_w || !off || !sorted || !y) return MOE_Q4_ERR_INVALID_ARG;
        for (const void* p : p4)
            if (!aligned(p, 4)) return MOE_Q4_ERR_INVALID_ARG;
        if (!aligned(y, 16)) return MOE_Q4_ERR_INVALID_ARG; // y is read and written as float4
    }
    for (const void* p : p16)
        if (p && !aligned(p, 16)) return MOE_Q4_ERR_INVALID_ARG;
    if ((int64_t)T * k > INT32_MAX / 2) return MOE_Q4_ERR_INVALID_ARG;
    if (E > MOE_Q4_MAX_EXPERTS || k > MOE_Q4_MAX_TOPK || !hidden_ok(H) || !inter_ok(I))
        return MOE_Q4_ERR_UNSUPPORTED;
    const size_t need = a16 ? moe_q4_prefill_a16_workspace_size(T, k, H, I) : moe_q4_workspace_size(T, E, k, H, I);
    if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256))) return MOE_Q4_ERR_WORKSPACE;
    return MOE_Q4_OK;
}

// The device scratch of moe_q4_decode_static: one copy per GPU, at its own
// device address.  In host code `scratch` names a host-side stand-in, never
// the device memory; every use goes through the address that
// hipGetSymbolAddress returns for the current device, obtained once per device.
static __device__ __align__(256) uint8_t scratch[MOE_Q4_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's scratch address, or nullptr (with *err set) on failure.
void* scratch_for_current_device(hipError_t* err)
{
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= MAX_DEVICES) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

} // namespace

extern "C" {

const char* moe_q4_status_string(int status)
{
    switch (status) {
    case MOE_Q4_OK: return "ok";
    case MOE_Q4_ERR_INVALID_ARG: return "invalid argument";
    case MOE_Q4_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_Q4_ERR_UNSUPPORTED: return "shape not supported by this build";
    case MOE_Q4_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

size_t moe_q4_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I)
{
    (void)E;
    if (T <= 0 || k <= 0 || I <= 0 || H <= 0) return 0;
    const size_t P = (size_t)T * (size_t)k;
    size_t n = WS_CTL_BYTES + align256(P * (size_t)I) + align256(P * (size_t)(I / 32) * sizeof(float));
    n += align256(P * (size_t)H * sizeof(float)); // per-pair o: decode's expert-major path, prefill's combine
    return n;
}

int moe_q4_quantize_act(const float* x, int64_t rows, int64_t cols, uint32_t flags, int8_t* xq, float* xd,
                        void* stream)
{
    if (rows < 0 || cols < 32 || cols % 32) return MOE_Q4_ERR_INVALID_ARG;
    if (cols > 16384 || rows > INT32_MAX) return MOE_Q4_ERR_UNSUPPORTED;
    if (flags & ~(uint32_t)MOE_Q4_QUANT_RMSNORM) return MOE_Q4_ERR_INVALID_ARG;
    if (rows == 0) return MOE_Q4_OK; // empty input: the pointers may be null
    if (!x || !xq || !xd) return MOE_Q4_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(xq, 4) || !aligned(xd, 4)) return MOE_Q4_ERR_INVALID_ARG;
    return hip_status(moeq4::launch_quantize_act(x, rows, (int)cols, (flags & MOE_Q4_QUANT_RMSNORM) != 0, xq, xd,
                                                 (hipStream_t)stream));
}

int moe_q4_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_w,
                 int32_t* expert_offsets, int32_t* sorted_pairs, void* stream)
{
    if (T < 0 || E < 1 || k < 1 || k > E) return MOE_Q4_ERR_INVALID_ARG;
    if (!expert_offsets || !aligned(expert_offsets, 4)) return MOE_Q4_ERR_INVALID_ARG;
    if (T > 0) { // with no tokens only expert_offsets is written (all zero)
        if (!logits || !topk_ids || !topk_w || !sorted_pairs) return MOE_Q4_ERR_INVALID_ARG;
        const void* p4[] = {logits, topk_ids, topk_w, sorted_pairs};
        for (const void* p : p4)
            if (!aligned(p, 4)) return MOE_Q4_ERR_INVALID_ARG;
    }
    if ((int64_t)T * k > INT32_MAX / 2) return MOE_Q4_ERR_INVALID_ARG;
    if (E > MOE_Q4_MAX_EXPERTS || k > MOE_Q4_MAX_TOPK) return MOE_Q4_ERR_UNSUPPORTED;
    return hip_status(moeq4::launch_route(logits, T, E, k, topk_ids, topk_w, expert_offsets, sorted_pairs,
                                          (hipStream_t)stream));
}

int moe_q4_decode(const moe_q4_experts* w, const int8_t* xq, const float* xd, int32_t T, int32_t k,
                  const int32_t* topk_ids, const float* topk_w, const int32_t* expert_offsets,
                  const int32_t* sorted_pairs, uint32_t flags, float* y, void* ws, size_t ws_bytes, void* stream)
{
    int rc = check_layer(w, xq, xd, T, k, topk_ids, topk_w, expert_offsets, sorted_pairs, flags, y, ws, ws_bytes);
    if (rc) return rc;
    if (T > MOE_Q4_MAX_DECODE_TOKENS) return MOE_Q4_ERR_UNSUPPORTED;
    const Ws s = carve(ws, (int64_t)T * k, w->hidden, w->inter);
    return hip_status(moeq4::launch_decode(w->gate_qs, w->up_qs, w->down_qs, w->gate_d, w->up_d, w->down_d,
                                           w->num_experts, w->hidden, w->inter, xq, xd, T, k, topk_w,
                                           expert_offsets, sorted_pairs, (flags & MOE_Q4_ACCUMULATE) != 0, y, s.hq,
                                           s.hd, s.o, (hipStream_t)stream));
}

int moe_q4_decode_static(const moe_q4_experts* w, const int8_t* xq, const float* xd, int32_t T, int32_t k,
                         const int32_t* topk_ids, const float* topk_w, const int32_t* expert_offsets,
                         const int32_t* sorted_pairs, uint32_t flags, float* y, void* stream)
{
    // the argument checks of moe_q4_decode, with a stand-in workspace of the scratch's size (not dereferenced)
    int rc = check_layer(w, xq, xd, T, k, topk_ids, topk_w, expert_offsets, sorted_pairs, flags, y,
                         reinterpret_cast<const void*>(uintptr_t(256)), MOE_Q4_STATIC_SCRATCH_BYTES);
    if (rc) return rc;
    if (T > MOE_Q4_MAX_DECODE_TOKENS) return MOE_Q4_ERR_UNSUPPORTED;
    if (T == 0) return MOE_Q4_OK;
    hipError_t err = hipSuccess;
    void* ws = scratch_for_current_device(&err);
    if (!ws) return MOE_Q4_ERR_HIP;
    const Ws s = carve(ws, (int64_t)T * k, w->hidden, w->inter);
    return hip_status(moeq4::launch_decode(w->gate_qs, w->up_qs, w->down_qs, w->gate_d, w->up_d, w->down_d,
                                           w->num_experts, w->hidden, w->inter, xq, xd, T, k, topk_w,
                                           expert_offsets, sorted_pairs, (flags & MOE_Q4_ACCUMULATE) != 0, y, s.hq,
                                           s.hd, s.o, (hipStream_t)stream));
}

int moe_q4_decode_fused(const moe_q4_experts* w, const float* x, const float* logits, int32_t T, int32_t k,
                        uint32_t flags, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                        int32_t* sorted_pairs, float* y, void* ws, size_t ws_bytes, void* stream)
{
    if (flags & ~(uint32_t)(MOE_Q4_QUANT_RMSNORM | MOE_Q4_ACCUMULATE)) return MOE_Q4_ERR_INVALID_ARG;
    // the layer checks (x stands in for xq/xd, which this call keeps on chip)
    int rc = check_layer(w, (const int8_t*)x, x, T, k, topk_ids, topk_w, expert_offsets, sorted_pairs,
                         flags & MOE_Q4_ACCUMULATE, y, ws, ws_bytes);
    if (rc) return rc;
    if (T == 0) return MOE_Q4_OK;
    if (!logits || !aligned(logits, 4)) return MOE_Q4_ERR_INVALID_ARG;
    if (!moeq4::fused_supported(T, k, w->inter)) return MOE_Q4_ERR_UNSUPPORTED;
    const Ws s = carve(ws, (int64_t)T * k, w->hidden, w->inter);
    return hip_status(moeq4::launch_decode_fused(
        w->gate_qs, w->up_qs, w->down_qs, w->gate_d, w->up_d, w->down_d, w->num_experts, w->hidden, w->inter, x,
        logits, T, k, (flags & MOE_Q4_QUANT_RMSNORM) != 0, (flags & MOE_Q4_ACCUMULATE) != 0, topk_ids, topk_w,
        expert_offsets, sorted_pairs, y, s.hq, s.hd, s.ctl, (hipStream_t)stream));
}

size_t moe_q4_stack_workspace_size(int32_t H)
{
    if (!hidden_ok(H)) return 0;
    return moeq4::stack_workspace_bytes(H);
}

int moe_q4_decode_stack(const moe_q4_experts* layers, int32_t L, const float* logits, int32_t k, uint32_t flags,
                        float* h, float* h_all, int8_t* hq_all, float* hd_all, void* ws, size_t ws_bytes,
                        void* stream)
{
    if (!layers || L < 1 || !logits || !h) return MOE_Q4_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)(MOE_Q4_QUANT_RMSNORM | MOE_Q4_ACCUMULATE)) return MOE_Q4_ERR_INVALID_ARG;
    if ((hq_all == nullptr) != (hd_all == nullptr)) return MOE_Q4_ERR_INVALID_ARG;
    const int E = layers[0].num_experts, H = layers[0].hidden, I = layers[0].inter;
    if (E < 1 || H <= 0 || I <= 0 || H % 32 || I % 32 || k < 1 || k > E) return MOE_Q4_ERR_INVALID_ARG;
    if (!aligned(h, 16) || !aligned(logits, 4) || (h_all && !aligned(h_all, 16)) || (hq_all && !aligned(hq_all, 16)) ||
        (hd_all && !aligned(hd_all, 4)))
        return MOE_Q4_ERR_INVALID_ARG;
    static_assert(MOE_Q4_MAX_STACK_LAYERS <= 64, "layer pointers travel as kernel arguments");
    const uint8_t* gq[MOE_Q4_MAX_STACK_LAYERS];
    const uint8_t* uq[MOE_Q4_MAX_STACK_LAYERS];
    const uint8_t* dq[MOE_Q4_MAX_STACK_LAYERS];
    const uint16_t* gd[MOE_Q4_MAX_STACK_LAYERS];
    const uint16_t* ud[MOE_Q4_MAX_STACK_LAYERS];
    const uint16_t* dd[MOE_Q4_MAX_STACK_LAYERS];
    if (L > MOE_Q4_MAX_STACK_LAYERS || L > moeq4::stack_max_layers()) return MOE_Q4_ERR_UNSUPPORTED;
    for (int l = 0; l < L; ++l) {
        const moe_q4_experts& w = layers[l];
        if (w.num_experts != E || w.hidden != H || w.inter != I) return MOE_Q4_ERR_INVALID_ARG;
        const void* p16[] = {w.gate_qs, w.up_qs, w.down_qs, w.gate_d, w.up_d, w.down_d};
        for (const void* p : p16)
            if (!p || !aligned(p, 16)) return MOE_Q4_ERR_INVALID_ARG;
        gq[l] = w.gate_qs;
        uq[l] = w.up_qs;
        dq[l] = w.down_qs;
        gd[l] = w.gate_d;
        ud[l] = w.up_d;
        dd[l] = w.down_d;
    }
    if (E > MOE_Q4_MAX_EXPERTS || !hidden_ok(H) || !moeq4::stack_supported(E, H, I, k)) return MOE_Q4_ERR_UNSUPPORTED;
    if (!ws || !aligned(ws, 256) || ws_bytes < moe_q4_stack_workspace_size(H)) return MOE_Q4_ERR_WORKSPACE;
    bool too_large = false;
    const hipError_t err = moeq4::launch_decode_stack(gq, uq, dq, gd, ud, dd, L, E, H, I, h, logits, k,
                                                      (flags & MOE_Q4_QUANT_RMSNORM) != 0,
                                                      (flags & MOE_Q4_ACCUMULATE) != 0, h_all, hq_all, hd_all, ws,
                                                      &too_large, (hipStream_t)stream);
    if (too_large) return MOE_Q4_ERR_UNSUPPORTED;
    return hip_status(err);
}

size_t moe_q4_stack_batch_workspace_size(int32_t L, int32_t T, int32_t E, int32_t k, int32_t H, int32_t I)
{
    if (L < 1 || L > moeq4::stack_batch_max_layers() || !moeq4::stack_batch_supported(E, H, I, T, k)) return 0;
    return moeq4::stack_batch_workspace_bytes(L, T, k, H, I);
}

int moe_q4_decode_stack_batch(const moe_q4_experts* layers, int32_t L, int32_t T, const float* logits, int32_t k,
                              uint32_t flags, float* h, float* h_all, int8_t* hq_all, float* hd_all, void* ws,
                              size_t ws_bytes, void* stream)
{
    if (!layers || L < 1 || T < 1 || !logits || !h) return MOE_Q4_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)(MOE_Q4_QUANT_RMSNORM | MOE_Q4_ACCUMULATE)) return MOE_Q4_ERR_INVALID_ARG;
    if ((hq_all == nullptr) != (hd_all == nullptr)) return MOE_Q4_ERR_INVALID_ARG;
    const int E = layers[0].num_experts, H = layers[0].hidden, I = layers[0].inter;
    if (E < 1 || H <= 0 || I <= 0 || H % 32 || I % 32 || k < 1 || k > E) return MOE_Q4_ERR_INVALID_ARG;
    if (!aligned(h, 16) || !aligned(logits, 4) || (h_all && !aligned(h_all, 16)) || (hq_all && !aligned(hq_all, 16)) ||
        (hd_all && !aligned(hd_all, 4)))
        return MOE_Q4_ERR_INVALID_ARG;
    if (L > MOE_Q4_MAX_STACK_LAYERS || L > moeq4::stack_batch_max_layers()) return MOE_Q4_ERR_UNSUPPORTED;
    const uint8_t* gq[MOE_Q4_MAX_STACK_LAYERS];
    const uint8_t* uq[MOE_Q4_MAX_STACK_LAYERS];
    const uint8_t* dq[MOE_Q4_MAX_STACK_LAYERS];
    const uint16_t* gd[MOE_Q4_MAX_STACK_LAYERS];
    const uint16_t* ud[MOE_Q4_MAX_STACK_LAYERS];
    const uint16_t* dd[MOE_Q4_MAX_STACK_LAYERS];
    for (int l = 0; l < L; ++l) {
        const moe_q4_experts& w = layers[l];
        if (w.num_experts != E || w.hidden != H || w.inter != I) return MOE_Q4_ERR_INVALID_ARG;
        const void* p16[] = {w.gate_qs, w.up_qs, w.down_qs, w.gate_d, w.up_d, w.down_d};
        for (const void* p : p16)
            if (!p || !aligned(p, 16)) return MOE_Q4_ERR_INVALID_ARG;
        gq[l] = w.gate_qs;
        uq[l] = w.up_qs;
        dq[l] = w.down_qs;
        gd[l] = w.gate_d;
        ud[l] = w.up_d;
        dd[l] = w.down_d;
    }
    if (E > MOE_Q4_MAX_EXPERTS || !moeq4::stack_batch_supported(E, H, I, T, k)) return MOE_Q4_ERR_UNSUPPORTED;
    const size_t need = moe_q4_stack_batch_workspace_size(L, T, E, k, H, I);
    if (!ws || !aligned(ws, 256) || ws_bytes < need) return MOE_Q4_ERR_WORKSPACE;
    bool too_large = false;
    const hipError_t err = moeq4::launch_decode_stack_batch(gq, uq, dq, gd, ud, dd, L, T, E, H, I, h, logits, k,
                                                            (flags & MOE_Q4_QUANT_RMSNORM) != 0,
                                                            (flags & MOE_Q4_ACCUMULATE) != 0, h_all, hq_all, hd_all,
                                                            ws, &too_large, (hipStream_t)stream);
    if (too_large) return MOE_Q4_ERR_UNSUPPORTED;
    return hip_status(err);
}

int moe_q4_prefill(const moe_q4_experts* w, const int8_t* xq, const float* xd, int32_t T, int32_t k,
                   const int32_t* topk_ids, const float* topk_w, const int32_t* expert_offsets,
                   const int32_t* sorted_pairs, uint32_t flags, float* y, void* ws, size_t ws_bytes, void* stream)
{
    int rc = check_layer(w, xq, xd, T, k, topk_ids, topk_w, expert_offsets, sorted_pairs, flags, y, ws, ws_bytes);
    if (rc) return rc;
    const Ws s = carve(ws, (int64_t)T * k, w->hidden, w->inter);
    return hip_status(moeq4::launch_prefill(w->gate_qs, w->up_qs, w->down_qs, w->gate_d, w->up_d, w->down_d,
                                            w->num_experts, w->hidden, w->inter, xq, xd, T, k, topk_w,
                                            expert_offsets, sorted_pairs, (flags & MOE_Q4_ACCUMULATE) != 0, y, s.hq,
                                            s.hd, s.o, (hipStream_t)stream));
}

size_t moe_q4_prefill_a16_workspace_size(int32_t T, int32_t k, int32_t H, int32_t I)
{
    if (T <= 0 || k <= 0 || I <= 0 || H <= 0) return 0;
    const size_t P = (size_t)T * (size_t)k;
    return align256((size_t)T * (size_t)H * 2) + align256(P * (size_t)I * 2) + align256(P * (size_t)H * sizeof(float));
}

int moe_q4_prefill_a16(const moe_q4_experts* w, const float* x, int32_t T, int32_t k, const int32_t* topk_ids,
                       const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_pairs, uint32_t flags,
                       float* y, void* ws, size_t ws_bytes, void* stream)
{
    // x takes the activations' place in the shared checks (16-byte aligned, fp32 rows)
    int rc = check_layer(w, reinterpret_cast<const int8_t*>(x), x, T, k, topk_ids, topk_w, expert_offsets, sorted_pairs,
                         flags, y, ws, ws_bytes, true);
    if (rc) return rc;
    if (T == 0) return MOE_Q4_OK;
    const int H = w->hidden, I = w->inter;
    _Float16* x16 = reinterpret_cast<_Float16*>(ws);
    _Float16* h16 = reinterpret_cast<_Float16*>((char*)ws + align256((size_t)T * H * 2));
    const size_t P = (size_t)T * (size_t)k;
    float* o = reinterpret_cast<float*>((char*)ws + align256((size_t)T * H * 2) + align256(P * (size_t)I * 2));
    return hip_status(moeq4::launch_prefill_a16(w->gate_qs, w->up_qs, w->down_qs, w->gate_d, w->up_d, w->down_d,
                                                w->num_experts, H, I, x, T, k, topk_w, expert_offsets, sorted_pairs,
                                                (flags & MOE_Q4_ACCUMULATE) != 0, y, x16, h16, o, (hipStream_t)stream));
}

int moe_q4_gemv(const uint8_t* qs, const uint16_t* d, int32_t N, int32_t K, const int8_t* xq, const float* xd,
                int32_t T, float* y, void* stream)
{
    if (N < 0 || T < 0) return MOE_Q4_ERR_INVALID_ARG;
    if (!hidden_ok(K) || T > MOE_Q4_MAX_DECODE_TOKENS) return MOE_Q4_ERR_UNSUPPORTED;
    if (N == 0 || T == 0) return MOE_Q4_OK; // empty: the pointers may be null
    if (!qs || !d || !xq || !xd || !y) return MOE_Q4_ERR_INVALID_ARG;
    if (!aligned(qs, 16) || !aligned(d, 16) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(y, 4))
        return MOE_Q4_ERR_INVALID_ARG;
    return hip_status(moeq4::launch_gemv(qs, d, N, K, xq, xd, T, y, (hipStream_t)stream));
}

int moe_q4_debug_block_dots(const uint8_t* qs, int32_t N, int32_t K, const int8_t* xq, int32_t T,
                            int32_t down_walk, int32_t* out, void* stream)
{
    if (!qs || !xq || !out || N < 0 || T < 0) return MOE_Q4_ERR_INVALID_ARG;
    if (!aligned(qs, 16) || !aligned(xq, 16) || !aligned(out, 4)) return MOE_Q4_ERR_INVALID_ARG;
    if (T > MOE_Q4_MAX_DECODE_TOKENS) return MOE_Q4_ERR_UNSUPPORTED;
    if (down_walk ? !inter_ok(K) : !hidden_ok(K)) return MOE_Q4_ERR_UNSUPPORTED;
    return hip_status(moeq4::launch_block_dots(qs, N, K, xq, T, down_walk != 0, out, (hipStream_t)stream));
}

int moe_q4_debug_prefill_dots(const moe_q4_experts* w, const int8_t* xq, const float* xd, int32_t T, int32_t k,
                              const int32_t* expert_offsets, const int32_t* sorted_pairs, int32_t which,
                              int32_t* out, void* ws, size_t ws_bytes, void* stream)
{
    if (!out || (which != 0 && which != 1)) return MOE_Q4_ERR_INVALID_ARG;
    // reuse the layer checks; topk ids/weights and y are not read here
    int rc = check_layer(w, xq, xd, T, k, expert_offsets, (const float*)expert_offsets, expert_offsets,
                         sorted_pairs, 0u, (const float*)out, ws, ws_bytes);
    if (rc) return rc;
    const Ws s = carve(ws, (int64_t)T * k, w->hidden, w->inter);
    return hip_status(moeq4::launch_prefill_dots(w->gate_qs, w->up_qs, w->down_qs, w->gate_d, w->up_d, w->down_d,
                                                 w->num_experts, w->hidden, w->inter, xq, xd, T, k, expert_offsets,
                                                 sorted_pairs, which, s.hq, s.hd, out, (hipStream_t)stream));
}

} // extern "C"
