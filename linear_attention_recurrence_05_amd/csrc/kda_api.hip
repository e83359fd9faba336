// kda_api.hip -- the C ABI declared in include/kda.h: argument validation
// (entirely on the host, before any HIP call), error reporting and dispatch
// to the kernel launchers.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/kda.h"
#include "kda_launch.hpp"

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

kda_status ok() {
    g_last_error.clear();
    return KDA_OK;
}

struct Range {
    const char* name;
    const void* p;
    size_t bytes;
    unsigned align;   // required alignment in bytes
};

bool overlap(const Range& a, const Range& b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Longest sequence: chunk counts and token offsets are formed in 32-bit ints.
constexpr int kMaxT = 1 << 30;

bool aligned(const void* p, unsigned a) { return ((uintptr_t)p & (uintptr_t)(a - 1)) == 0; }

kda_status check_common(int d_k, int d_v, kda_dtype dt, float g_min) {
    if (dt != KDA_F32 && dt != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "dtype %d is not KDA_F32 or KDA_BF16", (int)dt);
    if (!(d_k == d_v && (d_k == 32 || d_k == 128)))
        return fail(KDA_ERR_UNSUPPORTED, "(d_k, d_v) = (%d, %d); supported: (32, 32), (128, 128)", d_k, d_v);
    if (!std::isfinite(g_min) || g_min < -5.0f || g_min > 0.0f)
        return fail(KDA_ERR_INVALID_VALUE, "g_min = %g outside [-5, 0]", (double)g_min);
    return KDA_OK;
}

// Checks a list of tensor ranges for NULL (when required) and alignment.
kda_status check_ptrs(const Range* r, int n, const bool* required) {
    for (int i = 0; i < n; ++i) {
        if (!r[i].p) {
            if (required[i]) return fail(KDA_ERR_NULL_POINTER, "%s is NULL", r[i].name);
            continue;
        }
        if (!aligned(r[i].p, r[i].align))
            return fail(KDA_ERR_MISALIGNED, "%s is not %u-byte aligned", r[i].name, r[i].align);
    }
    return KDA_OK;
}

kda_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Shape check shared by prefill-style calls; returns element counts.
kda_status check_shape(int B, int T, int H, int d, size_t& n_tok_el, size_t& n_tok) {
    if (B < 1 || T < 1 || H < 1) return fail(KDA_ERR_INVALID_SHAPE, "B=%d T=%d H=%d must all be >= 1", B, T, H);
    if (T > kMaxT) return fail(KDA_ERR_INVALID_SHAPE, "T=%d is too large (limit 2^30)", T);
    const unsigned long long tok = (unsigned long long)B * (unsigned long long)T * (unsigned long long)H;
    if ((long long)B * H > (1LL << 26) || tok > (1ULL << 40))
        return fail(KDA_ERR_INVALID_SHAPE, "B*T*H = %llu is too large", tok);
    if ((long long)H * d > (1LL << 24))
        return fail(KDA_ERR_INVALID_SHAPE, "H*d = %lld is too large (limit 2^24)", (long long)H * d);
    n_tok = (size_t)tok;
    n_tok_el = n_tok * (size_t)d;
    return KDA_OK;
}

// Checks shared by the paged entry points: the pool, the slot tables and the
// tensors of a [B, T, H, d] call; o and the pool may overlap nothing else.
// Slot values live on the device and are not read here: a sequence whose
// slot lies outside [0, n_slots) is skipped by the kernels.
kda_status check_paged(const void* q, const void* k, const void* v, const void* z,
                       const float* beta, const float* A, const float* pool, int n_slots,
                       const int* slots_in, bool in_required, const int* slots_out,
                       bool out_required, const void* o, int B, int T, int H, int d,
                       kda_dtype dt, const void* ws, size_t ws_need) {
    size_t nel, ntok;
    kda_status s = check_shape(B, T, H, d, nel, ntok);
    if (s != KDA_OK) return s;
    if (n_slots < 1) return fail(KDA_ERR_INVALID_SHAPE, "n_slots=%d must be >= 1", n_slots);
    if ((long long)n_slots * H > (1LL << 26))
        return fail(KDA_ERR_INVALID_SHAPE, "n_slots*H = %lld is too large", (long long)n_slots * H);
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const Range r[] = {{"q", q, nel * es, 16},      {"k", k, nel * es, 16},
                       {"v", v, nel * es, 16},      {"z", z, nel * es, 16},
                       {"beta", beta, ntok * 4, 4}, {"A", A, (size_t)H * 4, 4},
                       {"slots_in", slots_in, (size_t)B * 4, 4},
                       {"slots_out", slots_out, (size_t)B * 4, 4},
                       {"pool", pool, (size_t)n_slots * H * d * d * sizeof(float), 16},
                       {"o", o, nel * es, 16},      {"workspace", ws, ws_need, 16}};
    const bool req[] = {true, true, true, true, true, true, in_required, out_required, true, true,
                        ws_need > 0};
    if ((s = check_ptrs(r, 11, req)) != KDA_OK) return s;
    for (int out : {8, 9, 10})
        for (int i = 0; i < 11; ++i)
            if (i != out && overlap(r[out], r[i]))
                return fail(KDA_ERR_ALIASING, "%s overlaps %s", r[out].name, r[i].name);
    return KDA_OK;
}

kda::StateIO paged_state(float* pool, int n_slots, const int* slots_in, const int* slots_out) {
    return kda::StateIO{slots_in ? pool : nullptr, slots_in, slots_out ? pool : nullptr, slots_out,
                        slots_in, slots_out, n_slots};
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL_POINTER: return "KDA_ERR_NULL_POINTER";
        case KDA_ERR_INVALID_SHAPE: return "KDA_ERR_INVALID_SHAPE";
        case KDA_ERR_INVALID_VALUE: return "KDA_ERR_INVALID_VALUE";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
        case KDA_ERR_ALIASING: return "KDA_ERR_ALIASING";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

// Workspace of the dense prefill: the segment scan's when it runs one, else
// the chosen plan's.
static size_t prefill_ws_bytes(int B, int T, int H, int d, bool is_bf16, int R) {
    return R > 1 ? kda::seg_layout(B, T, H, d, is_bf16, R).total
                 : kda::choose_plan(B, T, H, d, is_bf16).ws_bytes;
}

size_t kda_chunk_prefill_workspace_bytes(int B, int T, int H, int d_k, int d_v, kda_dtype dt) {
    size_t a, b;
    if (check_common(d_k, d_v, dt, -5.0f) != KDA_OK || check_shape(B, T, H, d_k, a, b) != KDA_OK) return 0;
    const bool bf = dt == KDA_BF16;
    return prefill_ws_bytes(B, T, H, d_k, bf, kda::auto_segments(B, T, H, d_k, bf));
}

int kda_chunk_prefill_segments(int B, int T, int H, int d_k, int d_v, kda_dtype dt) {
    size_t a, b;
    if (check_common(d_k, d_v, dt, -5.0f) != KDA_OK || check_shape(B, T, H, d_k, a, b) != KDA_OK) return 0;
    return kda::auto_segments(B, T, H, d_k, dt == KDA_BF16);
}

const char* kda_chunk_prefill_plan(int B, int T, int H, int d_k, int d_v, kda_dtype dt) {
    size_t a, b;
    if (check_common(d_k, d_v, dt, -5.0f) != KDA_OK || check_shape(B, T, H, d_k, a, b) != KDA_OK) return "";
    if (kda::auto_segments(B, T, H, d_k, dt == KDA_BF16) > 1) return "segment scan";
    const kda::PlanInfo p = kda::choose_plan(B, T, H, d_k, dt == KDA_BF16);
    if (p.plan == kda::Plan::kRing) return "ring";
    if (p.plan == kda::Plan::kSplit) return "split";
    switch (p.ncol) {
        case 16: return "fused:16";
        case 32: return "fused:32";
        case 64: return "fused:64";
        default: return "fused:128";
    }
}

}  // extern "C"

namespace {

// Static scratch of kda_chunk_prefill_noalloc: one copy per GPU, held until
// the process ends.  In host code `scratch` names a host-side stand-in; the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device (with that device current) and kept in g_scratch.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the scratch on the device `stream` runs on.
kda_status scratch_for(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KDA_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return fail(KDA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(KDA_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess)
            return fail(KDA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        if (e2 != hipSuccess)
            return fail(KDA_ERR_HIP, "hipSetDevice(%d): %s", cur, hipGetErrorString(e2));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KDA_OK;
}

// kda_chunk_prefill and kda_chunk_prefill_noalloc: validation (host only,
// before any HIP call), then the launch.  With use_scratch the workspace is
// the device's static scratch (the caller's workspace arguments are unused).
kda_status prefill_entry(const char* name, const void* q, const void* k, const void* v,
                         const void* z, const float* beta, const float* A, float g_min,
                         const float* S0, void* o, float* S_T, int B, int T, int H, int d_k,
                         int d_v, kda_dtype dt, void* workspace, size_t workspace_bytes,
                         void* stream, bool use_scratch) {
    kda_status s = check_common(d_k, d_v, dt, g_min);
    if (s != KDA_OK) return s;
    size_t nel, ntok;
    if ((s = check_shape(B, T, H, d_k, nel, ntok)) != KDA_OK) return s;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const size_t st_bytes = (size_t)B * H * d_k * d_v * sizeof(float);
    const bool bf = dt == KDA_BF16;
    const int nseg = kda::auto_segments(B, T, H, d_k, bf);
    const size_t need = prefill_ws_bytes(B, T, H, d_k, bf, nseg);
    if (use_scratch) {
        workspace = nullptr;   // the scratch overlaps no caller buffer
        if (need > KDA_NOALLOC_SCRATCH_BYTES)
            return fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                        "%s: these sizes need %zu bytes of scratch, the static scratch holds %zu "
                        "(call kda_chunk_prefill with a workspace instead)",
                        name, need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
    }
    const Range r[] = {{"q", q, nel * es, 16},          {"k", k, nel * es, 16},
                       {"v", v, nel * es, 16},          {"z", z, nel * es, 16},
                       {"beta", beta, ntok * 4, 4},     {"A", A, (size_t)H * 4, 4},
                       {"S0", S0, st_bytes, 4},         {"o", o, nel * es, 16},
                       {"S_T", S_T, st_bytes, 4},       {"workspace", workspace, need, 16}};
    const bool req[] = {true, true, true, true, true, true, false, true, false,
                        need > 0 && !use_scratch};
    if ((s = check_ptrs(r, 10, req)) != KDA_OK) return s;
    if (!use_scratch && workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    need);
    // outputs (o, S_T, workspace) against every other range; S_T == S0 exactly is allowed
    for (int out : {7, 8, 9}) {
        for (int i = 0; i < 10; ++i) {
            if (i == out) continue;
            if (out == 8 && i == 6 && S_T == S0) continue;
            if (overlap(r[out], r[i]))
                return fail(KDA_ERR_ALIASING, "%s overlaps %s", r[out].name, r[i].name);
        }
    }
    if (use_scratch && need > 0 && (s = scratch_for((hipStream_t)stream, &workspace)) != KDA_OK)
        return s;
    kda::PrefillArgs a{q, k, v, z, beta, A, g_min, kda::dense_state(S0, S_T), o, B, T, H, d_k,
                       dt == KDA_BF16};
    if (nseg > 1)
        return hip_status(kda::launch_segmented(a, nseg, workspace, (hipStream_t)stream),
                          "kda_chunk_prefill launch (segment scan)");
    const kda::PlanInfo plan = kda::choose_plan(B, T, H, d_k, bf);
    return hip_status(kda::launch_prefill(a, plan, workspace, (hipStream_t)stream), "kda_chunk_prefill launch");
}

}  // namespace

extern "C" {

kda_status kda_chunk_prefill(const void* q, const void* k, const void* v, const void* z,
                             const float* beta, const float* A, float g_min, const float* S0,
                             void* o, float* S_T, int B, int T, int H, int d_k, int d_v,
                             kda_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_entry("kda_chunk_prefill", q, k, v, z, beta, A, g_min, S0, o, S_T, B, T, H,
                         d_k, d_v, dt, workspace, workspace_bytes, stream, false);
}

kda_status kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const void* z,
                                     const float* beta, const float* A, float g_min,
                                     const float* S0, void* o, float* S_T, int B, int T, int H,
                                     int d_k, int d_v, kda_dtype dt, void* stream) {
    return prefill_entry("kda_chunk_prefill_noalloc", q, k, v, z, beta, A, g_min, S0, o, S_T, B,
                         T, H, d_k, d_v, dt, nullptr, 0, stream, true);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* z,
                           const float* beta, const float* A, float g_min, float* S, void* o,
                           int B, int H, int d_k, int d_v, kda_dtype dt, void* stream) {
    kda_status s = check_common(d_k, d_v, dt, g_min);
    if (s != KDA_OK) return s;
    size_t nel, ntok;
    if ((s = check_shape(B, 1, H, d_k, nel, ntok)) != KDA_OK) return s;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const Range r[] = {{"q", q, nel * es, 16},      {"k", k, nel * es, 16},   {"v", v, nel * es, 16},
                       {"z", z, nel * es, 16},      {"beta", beta, ntok * 4, 4},
                       {"A", A, (size_t)H * 4, 4},  {"S", S, (size_t)B * H * d_k * d_v * sizeof(float), 16},
                       {"o", o, nel * es, 16}};
    const bool req[] = {true, true, true, true, true, true, true, true};
    if ((s = check_ptrs(r, 8, req)) != KDA_OK) return s;
    for (int out : {6, 7})
        for (int i = 0; i < 8; ++i)
            if (i != out && overlap(r[out], r[i]))
                return fail(KDA_ERR_ALIASING, "%s overlaps %s", r[out].name, r[i].name);
    kda::DecodeArgs a{q, k, v, z, beta, A, g_min, kda::dense_state(S, S), o, B, H, d_k, dt == KDA_BF16};
    return hip_status(kda::launch_decode(a, (hipStream_t)stream), "kda_decode_step launch");
}

kda_status kda_decode_tokens(const void* q, const void* k, const void* v, const void* z,
                             const float* beta, const float* A, float g_min, const float* S,
                             float* S_out, void* o, int B, int T, int H, int d_k, int d_v,
                             kda_dtype dt, void* stream) {
    kda_status s = check_common(d_k, d_v, dt, g_min);
    if (s != KDA_OK) return s;
    if (T < 1 || T > KDA_MAX_DECODE_TOKENS)
        return fail(KDA_ERR_INVALID_SHAPE, "T=%d outside [1, %d]", T, KDA_MAX_DECODE_TOKENS);
    size_t nel, ntok;
    if ((s = check_shape(B, T, H, d_k, nel, ntok)) != KDA_OK) return s;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const size_t sbytes = (size_t)B * H * d_k * d_v * sizeof(float);
    const Range r[] = {{"q", q, nel * es, 16},     {"k", k, nel * es, 16},
                       {"v", v, nel * es, 16},     {"z", z, nel * es, 16},
                       {"beta", beta, ntok * 4, 4}, {"A", A, (size_t)H * 4, 4},
                       {"S", S, sbytes, 16},       {"S_out", S_out, sbytes, 16},
                       {"o", o, nel * es, 16}};
    const bool req[] = {true, true, true, true, true, true, true, true, true};
    if ((s = check_ptrs(r, 9, req)) != KDA_OK) return s;
    // S_out may be S itself (commit in place) but may not overlap it partly;
    // o and S_out may not overlap anything else
    for (int out : {7, 8})
        for (int i = 0; i < 9; ++i) {
            if (i == out || (out == 7 && i == 6 && S_out == S)) continue;
            if (overlap(r[out], r[i])) return fail(KDA_ERR_ALIASING, "%s overlaps %s", r[out].name, r[i].name);
        }
    kda::TokensArgs a{q, k, v, z, beta, A, g_min, kda::dense_state(S, S_out), o, B, T, H, d_k,
                      dt == KDA_BF16};
    return hip_status(kda::launch_tokens(a, (hipStream_t)stream), "kda_decode_tokens launch");
}

size_t kda_chunk_prefill_paged_workspace_bytes(int B, int T, int H, int d_k, int d_v,
                                               kda_dtype dt) {
    size_t a, b;
    if (check_common(d_k, d_v, dt, -5.0f) != KDA_OK || check_shape(B, T, H, d_k, a, b) != KDA_OK) return 0;
    return kda::choose_plan(B, T, H, d_k, dt == KDA_BF16).ws_bytes;
}

kda_status kda_chunk_prefill_paged(const void* q, const void* k, const void* v, const void* z,
                                   const float* beta, const float* A, float g_min, float* pool,
                                   int n_slots, const int* slots_in, const int* slots_out, void* o,
                                   int B, int T, int H, int d_k, int d_v, kda_dtype dt,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    kda_status s = check_common(d_k, d_v, dt, g_min);
    if (s != KDA_OK) return s;
    size_t nel, ntok;
    if ((s = check_shape(B, T, H, d_k, nel, ntok)) != KDA_OK) return s;
    const kda::PlanInfo plan = kda::choose_plan(B, T, H, d_k, dt == KDA_BF16);
    if ((s = check_paged(q, k, v, z, beta, A, pool, n_slots, slots_in, false, slots_out, false, o, B,
                         T, H, d_k, dt, workspace, plan.ws_bytes)) != KDA_OK)
        return s;
    if (workspace_bytes < plan.ws_bytes)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                    "workspace of %zu bytes, %zu needed (kda_chunk_prefill_paged_workspace_bytes)",
                    workspace_bytes, plan.ws_bytes);
    kda::PrefillArgs a{q, k, v, z, beta, A, g_min, paged_state(pool, n_slots, slots_in, slots_out), o,
                       B, T, H, d_k, dt == KDA_BF16};
    return hip_status(kda::launch_prefill(a, plan, workspace, (hipStream_t)stream),
                      "kda_chunk_prefill_paged launch");
}

kda_status kda_decode_step_paged(const void* q, const void* k, const void* v, const void* z,
                                 const float* beta, const float* A, float g_min, float* pool,
                                 int n_slots, const int* slots, void* o, int B, int H, int d_k,
                                 int d_v, kda_dtype dt, void* stream) {
    kda_status s = check_common(d_k, d_v, dt, g_min);
    if (s != KDA_OK) return s;
    if ((s = check_paged(q, k, v, z, beta, A, pool, n_slots, slots, true, slots, true, o, B, 1, H, d_k,
                         dt, nullptr, 0)) != KDA_OK)
        return s;
    kda::DecodeArgs a{q, k, v, z, beta, A, g_min, paged_state(pool, n_slots, slots, slots), o, B, H,
                      d_k, dt == KDA_BF16};
    return hip_status(kda::launch_decode(a, (hipStream_t)stream), "kda_decode_step_paged launch");
}

kda_status kda_decode_tokens_paged(const void* q, const void* k, const void* v, const void* z,
                                   const float* beta, const float* A, float g_min, float* pool,
                                   int n_slots, const int* slots_in, const int* slots_out, void* o,
                                   int B, int T, int H, int d_k, int d_v, kda_dtype dt,
                                   void* stream) {
    kda_status s = check_common(d_k, d_v, dt, g_min);
    if (s != KDA_OK) return s;
    if (T < 1 || T > KDA_MAX_DECODE_TOKENS)
        return fail(KDA_ERR_INVALID_SHAPE, "T=%d outside [1, %d]", T, KDA_MAX_DECODE_TOKENS);
    if ((s = check_paged(q, k, v, z, beta, A, pool, n_slots, slots_in, true, slots_out, true, o, B, T,
                         H, d_k, dt, nullptr, 0)) != KDA_OK)
        return s;
    kda::TokensArgs a{q, k, v, z, beta, A, g_min, paged_state(pool, n_slots, slots_in, slots_out), o,
                      B, T, H, d_k, dt == KDA_BF16};
    return hip_status(kda::launch_tokens(a, (hipStream_t)stream), "kda_decode_tokens_paged launch");
}

size_t kda_chunk_prefill_segmented_workspace_bytes(int B, int T, int H, int d_k, int d_v,
                                                   int n_seg, kda_dtype dt) {
    if (dt != KDA_F32 && dt != KDA_BF16) return 0;
    if (!(d_k == d_v && (d_k == 32 || d_k == 128))) return 0;
    if (B < 1 || T < 1 || H < 1 || T > kMaxT || n_seg < 1 || T % n_seg != 0 ||
        (long long)B * n_seg * H > (1LL << 26) || (unsigned long long)B * T * H > (1ULL << 40) ||
        (long long)H * d_k > (1LL << 24))
        return 0;
    return kda::seg_layout(B, T, H, d_k, dt == KDA_BF16, n_seg).total;
}

kda_status kda_chunk_prefill_segmented(const void* q, const void* k, const void* v, const void* z,
                                       const float* beta, const float* A, float g_min,
                                       const float* S0, void* o, float* S_T, int B, int T, int H,
                                       int d_k, int d_v, int n_seg, kda_dtype dt, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    kda_status s = check_common(d_k, d_v, dt, g_min);
    if (s != KDA_OK) return s;
    size_t nel, ntok;
    if ((s = check_shape(B, T, H, d_k, nel, ntok)) != KDA_OK) return s;
    if (n_seg < 1 || T % n_seg != 0)
        return fail(KDA_ERR_INVALID_SHAPE, "n_seg=%d must be >= 1 and divide T=%d", n_seg, T);
    if ((long long)B * n_seg * H > (1LL << 26))
        return fail(KDA_ERR_INVALID_SHAPE, "B*n_seg*H = %lld is too large", (long long)B * n_seg * H);
    const size_t need = kda::seg_layout(B, T, H, d_k, dt == KDA_BF16, n_seg).total;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const size_t st_bytes = (size_t)B * H * d_k * d_v * sizeof(float);
    const Range r[] = {{"q", q, nel * es, 16},          {"k", k, nel * es, 16},
                       {"v", v, nel * es, 16},          {"z", z, nel * es, 16},
                       {"beta", beta, ntok * 4, 4},     {"A", A, (size_t)H * 4, 4},
                       {"S0", S0, st_bytes, 4},         {"o", o, nel * es, 16},
                       {"S_T", S_T, st_bytes, 4},       {"workspace", workspace, need, 16}};
    const bool req[] = {true, true, true, true, true, true, false, true, false, true};
    if ((s = check_ptrs(r, 10, req)) != KDA_OK) return s;
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    for (int out : {7, 8, 9}) {
        for (int i = 0; i < 10; ++i) {
            if (i == out) continue;
            if (out == 8 && i == 6 && S_T == S0) continue;
            if (overlap(r[out], r[i]))
                return fail(KDA_ERR_ALIASING, "%s overlaps %s", r[out].name, r[i].name);
        }
    }
    kda::PrefillArgs a{q, k, v, z, beta, A, g_min, kda::dense_state(S0, S_T), o, B, T, H, d_k,
                       dt == KDA_BF16};
    return hip_status(kda::launch_segmented(a, n_seg, workspace, (hipStream_t)stream),
                      "kda_chunk_prefill_segmented launch");
}

size_t kda_chunk_backward_workspace_bytes(int B, int T, int H, int d_k, int d_v, kda_dtype dt) {
    if (dt != KDA_F32 && dt != KDA_BF16) return 0;
    if (!(d_k == d_v && (d_k == 32 || d_k == 128))) return 0;
    if (B < 1 || T < 1 || H < 1 || T > kMaxT || (long long)B * H > (1LL << 26) ||
        (unsigned long long)B * T * H > (1ULL << 40) || (long long)H * d_k > (1LL << 24))
        return 0;
    return kda::bwd_layout(B, T, H, d_k, dt == KDA_BF16).total;
}

kda_status kda_chunk_backward(const void* q, const void* k, const void* v, const void* z,
                              const float* beta, const float* A, float g_min, const float* S0,
                              const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                              void* dz, float* dbeta, float* dA, float* dS0, int B, int T, int H,
                              int d_k, int d_v, kda_dtype dt, void* workspace,
                              size_t workspace_bytes, void* stream) {
    kda_status s = check_common(d_k, d_v, dt, g_min);
    if (s != KDA_OK) return s;
    size_t nel, ntok;
    if ((s = check_shape(B, T, H, d_k, nel, ntok)) != KDA_OK) return s;
    const size_t need = kda::bwd_layout(B, T, H, d_k, dt == KDA_BF16).total;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const size_t sbytes = (size_t)B * H * d_k * d_v * sizeof(float);
    const Range r[] = {{"q", q, nel * es, 16},       {"k", k, nel * es, 16},
                       {"v", v, nel * es, 16},       {"z", z, nel * es, 16},
                       {"beta", beta, ntok * 4, 4},  {"A", A, (size_t)H * 4, 4},
                       {"S0", S0, sbytes, 16},       {"dO", dO, nel * es, 16},
                       {"dS_T", dS_T, sbytes, 16},   {"dq", dq, nel * es, 16},
                       {"dk", dk, nel * es, 16},     {"dv", dv, nel * es, 16},
                       {"dz", dz, nel * es, 16},     {"dbeta", dbeta, ntok * 4, 4},
                       {"dA", dA, (size_t)H * 4, 4}, {"dS0", dS0, sbytes, 16},
                       {"workspace", workspace, need, 16}};
    constexpr int n = 17;
    const bool req[n] = {true, true, true, true, true, true, false, true, false,
                         true, true, true, true, true, true, false, true};
    if ((s = check_ptrs(r, n, req)) != KDA_OK) return s;
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    // outputs (dq .. dS0) and the workspace may overlap nothing else
    for (int out = 9; out < n; ++out)
        for (int i = 0; i < n; ++i)
            if (i != out && overlap(r[out], r[i]))
                return fail(KDA_ERR_ALIASING, "%s overlaps %s", r[out].name, r[i].name);
    kda::BackwardArgs a{q,  k,  v,  z,     beta, A,  g_min, S0, dO, dS_T, dq, dk,
                        dv, dz, dbeta, dA, dS0,  B,  T,     H,  d_k, dt == KDA_BF16};
    return hip_status(kda::launch_backward(a, workspace, (hipStream_t)stream),
                      "kda_chunk_backward launch");
}

kda_status kda_gate_chunk_cumsum(const void* z, const float* A, float g_min, float* G, int B, int T,
                                 int H, int d_k, kda_dtype dt, void* stream) {
    kda_status s = check_common(d_k, d_k, dt, g_min);
    if (s != KDA_OK) return s;
    size_t nel, ntok;
    if ((s = check_shape(B, T, H, d_k, nel, ntok)) != KDA_OK) return s;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const Range r[] = {{"z", z, nel * es, 16}, {"A", A, (size_t)H * 4, 4}, {"G", G, nel * 4, 4}};
    const bool req[] = {true, true, true};
    if ((s = check_ptrs(r, 3, req)) != KDA_OK) return s;
    if (overlap(r[2], r[0]) || overlap(r[2], r[1])) return fail(KDA_ERR_ALIASING, "G overlaps an input");
    return hip_status(kda::launch_gate_cumsum(z, A, g_min, G, B, T, H, d_k, dt == KDA_BF16, (hipStream_t)stream),
                      "kda_gate_chunk_cumsum launch");
}

kda_status kda_intra_chunk(const void* q, const void* k, const void* z, const float* beta,
                           const float* A, float g_min, float* Tm, float* Aqk, float* gamma, int B,
                           int T, int H, int d_k, kda_dtype dt, void* stream) {
    kda_status s = check_common(d_k, d_k, dt, g_min);
    if (s != KDA_OK) return s;
    size_t nel, ntok;
    if ((s = check_shape(B, T, H, d_k, nel, ntok)) != KDA_OK) return s;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const size_t nchunk = (size_t)B * H * ((T + KDA_CHUNK - 1) / KDA_CHUNK);
    const Range r[] = {{"q", q, nel * es, 16},       {"k", k, nel * es, 16},         {"z", z, nel * es, 16},
                       {"beta", beta, ntok * 4, 4}, {"A", A, (size_t)H * 4, 4},    {"Tm", Tm, nchunk * 1024, 4},
                       {"Aqk", Aqk, nchunk * 1024, 4}, {"gamma", gamma, nchunk * d_k * 4, 4}};
    const bool req[] = {true, true, true, true, true, true, true, true};
    if ((s = check_ptrs(r, 8, req)) != KDA_OK) return s;
    for (int out : {5, 6, 7})
        for (int i = 0; i < 8; ++i)
            if (i != out && overlap(r[out], r[i]))
                return fail(KDA_ERR_ALIASING, "%s overlaps %s", r[out].name, r[i].name);
    return hip_status(kda::launch_intra_diag(q, k, z, beta, A, g_min, Tm, Aqk, gamma, B, T, H, d_k,
                                             dt == KDA_BF16, (hipStream_t)stream),
                      "kda_intra_chunk launch");
}

}  // extern "C"
