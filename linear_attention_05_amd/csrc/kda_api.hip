// kda_api.hip -- the C ABI (include/kda.h): host-side validation, workspace
// sizing and launch of the gfx950 kernels. No HIP call happens before every
// argument has been validated.
#include "kda.h"

#include "kda_internal.h"

#include <atomic>
#include <cstring>
#include <mutex>

namespace kda {

DeviceInfo device_info() {
    constexpr int kMaxDevices = 64;
    static std::atomic<bool> ready[kMaxDevices];
    static DeviceInfo info[kMaxDevices];
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DeviceInfo{};
    if (ready[dev].load(std::memory_order_acquire)) return info[dev];
    std::lock_guard<std::mutex> lock(mu);
    if (!ready[dev].load(std::memory_order_relaxed)) {
        DeviceInfo d;
        int n = 0;
        bool ok = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0;
        if (ok) d.cus = n;
        ok = ok && hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && n > 0;
        if (ok) d.lds_per_block = n;
        ok = ok && hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess && n > 0;
        if (ok) d.lds_per_cu = n;
        d.valid = ok;
        if (!ok) return d;  // not cached: asked again next time
        info[dev] = d;
        ready[dev].store(true, std::memory_order_release);
    }
    return info[dev];
}

// ---- scratch of the allocation-free prefill entry point ----------------
// The workspace of kda_prefill_chunked_noalloc: a fixed device array of the
// library's code object (each device holds its own copy until the process
// ends). Host code never uses its name as an address: the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<bool> g_scratch_ready[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

// Device address of the current device's scratch (nullptr on failure).
void* scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    if (g_scratch_ready[dev].load(std::memory_order_acquire)) return g_scratch_ptr[dev];
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ready[dev].load(std::memory_order_relaxed)) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
        g_scratch_ready[dev].store(true, std::memory_order_release);
    }
    return g_scratch_ptr[dev];
}

}  // namespace kda

namespace {

constexpr int kVersion = 300;  // 0.3.0

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_dim(int32_t d) { return d == 64 || d == 128; }

// The bits of an enum argument, read without an enum-typed load: a C caller
// may pass any int where the ABI names an enum, and C++ gives an enum object
// holding a value outside its enumerators no defined value.
template <typename E>
int enum_bits(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "the C enums of kda.h are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

bool valid_dtype(int t) { return t == KDA_F32 || t == KDA_BF16; }

constexpr uint32_t kFrontMask = KDA_FRONT_L2NORM_QK | KDA_FRONT_GATE | KDA_FRONT_BETA_SIGMOID;
static_assert(KDA_FRONT_L2NORM_QK == kda::kFrontL2 && KDA_FRONT_GATE == kda::kFrontGate &&
                  KDA_FRONT_BETA_SIGMOID == kda::kFrontBeta,
              "front-end bits of kda.h and the kernels differ");

// Shared size checks of the prefill entry points (sizes only, no pointers).
kda_status_t check_prefill_sizes(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t Dk,
                                 int32_t Dv, int32_t chunk_size, int dt) {
    if (total_tokens < 0 || num_seqs < 1 || H < 1 || Dk < 1 || Dv < 1 || !valid_dtype(dt))
        return KDA_ERR_INVALID_ARG;
    if (total_tokens > (int64_t)INT32_MAX || (int64_t)num_seqs * H > (int64_t)INT32_MAX / 16)
        return KDA_ERR_UNSUPPORTED;
    if (!supported_dim(Dk) || !supported_dim(Dv) || chunk_size != kda::kChunk)
        return KDA_ERR_UNSUPPORTED;
    // the kernels address a chunk's rows with 32-bit offsets (r * H * D, r < 64)
    if ((int64_t)H * (Dk > Dv ? Dk : Dv) * kda::kChunk > (int64_t)INT32_MAX)
        return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_version(void) { return kVersion; }

const char* kda_status_string(kda_status_t s) {
    switch (enum_bits(s)) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: unsupported size or option";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP launch or runtime failure";
    }
    return "unknown kda_status_t";
}

size_t kda_prefill_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t Dk,
                                  int32_t Dv, int32_t chunk_size, kda_dtype_t in_dtype) {
    const int dt = enum_bits(in_dtype);
    if (check_prefill_sizes(total_tokens, num_seqs, H, Dk, Dv, chunk_size, dt) != KDA_OK)
        return 0;
    const bool bf16 = dt == KDA_BF16;
    const size_t plain = kda::prefill_workspace_bytes(total_tokens, num_seqs, H, Dk, Dv, bf16);
    const size_t split = kda::prefill_split_workspace_bytes(total_tokens, num_seqs, H, Dk, Dv, bf16);
    return plain > split ? plain : split;
}

int32_t kda_prefill_scan_segments(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t Dk,
                                  int32_t Dv, int32_t chunk_size, kda_dtype_t in_dtype) {
    const int dt = enum_bits(in_dtype);
    if (check_prefill_sizes(total_tokens, num_seqs, H, Dk, Dv, chunk_size, dt) != KDA_OK)
        return 0;
    const kda::DeviceInfo di = kda::device_info();
    if (!di.valid) return 1;
    const int cus = di.cus;
    const bool bf16 = dt == KDA_BF16;
    const int want = kda::prefill_split_segments(total_tokens, num_seqs, H, Dk, Dv, bf16, cus);
    const int sized = kda::prefill_split_segments(total_tokens, num_seqs, H, Dk, Dv, bf16, kda::kSizingCUs);
    const int P = want < sized ? want : sized;
    return P < 2 ? 1 : P;
}

}  // extern "C"

namespace {

// Validation (host only, before any HIP call) and launch of every prefill
// entry point. use_scratch: the workspace is the library's static scratch,
// looked up only after every argument has passed.
kda_status_t prefill_impl(const void* q, const void* k, const void* v, int dt,
                          const float* g, const float* beta, const int32_t* cu_seqlens,
                          int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t Dk,
                          int32_t Dv, int32_t chunk_size, const float* initial_state,
                          float* final_state, int64_t ckpt_interval, float* ckpt_states,
                          int64_t ckpt_rows, float* o, const int32_t* pos_offsets,
                          const int32_t* pos_values, int32_t num_pos, float* pos_states,
                          void* workspace, size_t workspace_bytes, bool use_scratch,
                          uint32_t phases, uint32_t frontend, hipStream_t stream) {
    if (phases == 0 || (phases & ~(KDA_PHASE_PREPARE | KDA_PHASE_SCAN)) != 0)
        return KDA_ERR_INVALID_ARG;
    if (frontend & ~kFrontMask) return KDA_ERR_INVALID_ARG;
    if (num_pos < 0) return KDA_ERR_INVALID_ARG;
    if (num_pos > 0) {
        if (!pos_offsets || !pos_values || !pos_states) return KDA_ERR_INVALID_ARG;
        if (!aligned(pos_offsets, 4) || !aligned(pos_values, 4) || !aligned(pos_states, 16))
            return KDA_ERR_INVALID_ARG;
        if ((int64_t)num_pos * H * 4 > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;  // advance grid
    }
    kda_status_t st = check_prefill_sizes(total_tokens, num_seqs, H, Dk, Dv, chunk_size, dt);
    if (st != KDA_OK) return st;
    if (!cu_seqlens && num_seqs != 1) return KDA_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_INVALID_ARG;
    if (ckpt_interval < 0) return KDA_ERR_INVALID_ARG;
    if (ckpt_interval > 0 && (ckpt_interval % chunk_size != 0)) return KDA_ERR_UNSUPPORTED;
    if (ckpt_interval > 0 && (!ckpt_states || ckpt_rows < 0)) return KDA_ERR_INVALID_ARG;
    if (ckpt_interval == 0 && (ckpt_states || ckpt_rows != 0)) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, g, beta, cu_seqlens, initial_state, final_state, ckpt_states, o};
    for (const void* p : ptrs)
        if (p && !aligned(p, 16)) return KDA_ERR_INVALID_ARG;
    const size_t need =
        kda::prefill_workspace_bytes(total_tokens, num_seqs, H, Dk, Dv, dt == KDA_BF16);
    if (use_scratch) {
        if (need > kda::kScratchBytes) return KDA_ERR_WORKSPACE;
        workspace = kda::scratch_address();  // the first HIP call
        workspace_bytes = kda::kScratchBytes;
        if (!workspace) return KDA_ERR_HIP;
    }
    if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return KDA_ERR_INVALID_ARG;

    kda::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.bf16 = dt == KDA_BF16;
    a.g = g;
    a.beta = beta;
    a.cu_seqlens = cu_seqlens;
    a.num_seqs = num_seqs;
    a.total_tokens = total_tokens;
    a.H = H;
    a.Dk = Dk;
    a.Dv = Dv;
    a.initial_state = initial_state;
    a.final_state = final_state;
    a.ckpt_interval = ckpt_interval;
    a.ckpt_states = ckpt_states;
    a.ckpt_rows = ckpt_rows;
    a.o = o;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    a.phases = phases;
    a.frontend = frontend;
    if (num_pos > 0) {
        a.pos.offsets = pos_offsets;
        a.pos.values = pos_values;
        a.pos.states = pos_states;
        a.pos.num_pos = num_pos;
    }
    return kda::launch_prefill(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

kda_status_t kda_prefill_chunked_at(const void* q, const void* k, const void* v,
                                    kda_dtype_t in_dtype, const float* g, const float* beta,
                                    const int32_t* cu_seqlens, int32_t num_seqs,
                                    int64_t total_tokens, int32_t H, int32_t Dk, int32_t Dv,
                                    int32_t chunk_size, const float* initial_state,
                                    float* final_state, int64_t ckpt_interval,
                                    float* ckpt_states, int64_t ckpt_rows, float* o,
                                    const int32_t* pos_offsets, const int32_t* pos_values,
                                    int32_t num_pos, float* pos_states, void* workspace,
                                    size_t workspace_bytes, uint32_t phases, uint32_t frontend,
                                    hipStream_t stream) {
    return prefill_impl(q, k, v, enum_bits(in_dtype), g, beta, cu_seqlens, num_seqs, total_tokens,
                        H, Dk, Dv, chunk_size, initial_state, final_state, ckpt_interval,
                        ckpt_states, ckpt_rows, o, pos_offsets, pos_values, num_pos, pos_states,
                        workspace, workspace_bytes, false, phases, frontend, stream);
}

kda_status_t kda_prefill_chunked_ex(const void* q, const void* k, const void* v,
                                    kda_dtype_t in_dtype, const float* g, const float* beta,
                                    const int32_t* cu_seqlens, int32_t num_seqs,
                                    int64_t total_tokens, int32_t H, int32_t Dk, int32_t Dv,
                                    int32_t chunk_size, const float* initial_state,
                                    float* final_state, int64_t ckpt_interval,
                                    float* ckpt_states, int64_t ckpt_rows, float* o,
                                    void* workspace, size_t workspace_bytes, uint32_t phases,
                                    uint32_t frontend, hipStream_t stream) {
    return prefill_impl(q, k, v, enum_bits(in_dtype), g, beta, cu_seqlens, num_seqs, total_tokens,
                        H, Dk, Dv, chunk_size, initial_state, final_state, ckpt_interval,
                        ckpt_states, ckpt_rows, o, nullptr, nullptr, 0, nullptr, workspace,
                        workspace_bytes, false, phases, frontend, stream);
}

kda_status_t kda_prefill_chunked_phases(const void* q, const void* k, const void* v,
                                        kda_dtype_t in_dtype, const float* g, const float* beta,
                                        const int32_t* cu_seqlens, int32_t num_seqs,
                                        int64_t total_tokens, int32_t H, int32_t Dk, int32_t Dv,
                                        int32_t chunk_size, const float* initial_state,
                                        float* final_state, int64_t ckpt_interval,
                                        float* ckpt_states, int64_t ckpt_rows, float* o,
                                        void* workspace, size_t workspace_bytes, uint32_t phases,
                                        hipStream_t stream) {
    return prefill_impl(q, k, v, enum_bits(in_dtype), g, beta, cu_seqlens, num_seqs, total_tokens,
                        H, Dk, Dv, chunk_size, initial_state, final_state, ckpt_interval,
                        ckpt_states, ckpt_rows, o, nullptr, nullptr, 0, nullptr, workspace,
                        workspace_bytes, false, phases, 0u, stream);
}

kda_status_t kda_prefill_chunked(const void* q, const void* k, const void* v,
                                 kda_dtype_t in_dtype, const float* g, const float* beta,
                                 const int32_t* cu_seqlens, int32_t num_seqs,
                                 int64_t total_tokens, int32_t H, int32_t Dk, int32_t Dv,
                                 int32_t chunk_size, const float* initial_state,
                                 float* final_state, int64_t ckpt_interval, float* ckpt_states,
                                 int64_t ckpt_rows, float* o, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    return prefill_impl(q, k, v, enum_bits(in_dtype), g, beta, cu_seqlens, num_seqs, total_tokens,
                        H, Dk, Dv, chunk_size, initial_state, final_state, ckpt_interval,
                        ckpt_states, ckpt_rows, o, nullptr, nullptr, 0, nullptr, workspace,
                        workspace_bytes, false, KDA_PHASE_PREPARE | KDA_PHASE_SCAN, 0u, stream);
}

kda_status_t kda_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                         kda_dtype_t in_dtype, const float* g, const float* beta,
                                         const int32_t* cu_seqlens, int32_t num_seqs,
                                         int64_t total_tokens, int32_t H, int32_t Dk, int32_t Dv,
                                         int32_t chunk_size, const float* initial_state,
                                         float* final_state, int64_t ckpt_interval,
                                         float* ckpt_states, int64_t ckpt_rows, float* o,
                                         hipStream_t stream) {
    return prefill_impl(q, k, v, enum_bits(in_dtype), g, beta, cu_seqlens, num_seqs, total_tokens,
                        H, Dk, Dv, chunk_size, initial_state, final_state, ckpt_interval,
                        ckpt_states, ckpt_rows, o, nullptr, nullptr, 0, nullptr, nullptr, 0, true,
                        KDA_PHASE_PREPARE | KDA_PHASE_SCAN, 0u, stream);
}

}  // extern "C"

namespace {

kda_status_t decode_impl(const void* q, const void* k, const void* v, int dt, const float* g,
                         const float* beta, int32_t B, int32_t H, int32_t Dk, int32_t Dv,
                         float* state, float* o, uint32_t frontend, hipStream_t stream) {
    if (frontend & ~kFrontMask) return KDA_ERR_INVALID_ARG;
    if (B < 0 || H < 1 || Dk < 1 || Dv < 1 || !valid_dtype(dt)) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)B * H > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (B == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, g, beta, state, o};
    for (const void* p : ptrs)
        if (!aligned(p, 16)) return KDA_ERR_INVALID_ARG;
    return kda::launch_decode(q, k, v, dt == KDA_BF16, g, beta, B, H, Dk, Dv, state, o,
                              frontend, stream) == hipSuccess
               ? KDA_OK
               : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

kda_status_t kda_decode_step_ex(const void* q, const void* k, const void* v,
                                kda_dtype_t in_dtype, const float* g, const float* beta,
                                int32_t B, int32_t H, int32_t Dk, int32_t Dv, float* state,
                                float* o, uint32_t frontend, hipStream_t stream) {
    return decode_impl(q, k, v, enum_bits(in_dtype), g, beta, B, H, Dk, Dv, state, o, frontend,
                       stream);
}

kda_status_t kda_decode_step(const void* q, const void* k, const void* v, kda_dtype_t in_dtype,
                             const float* g, const float* beta, int32_t B, int32_t H, int32_t Dk,
                             int32_t Dv, float* state, float* o, hipStream_t stream) {
    return decode_impl(q, k, v, enum_bits(in_dtype), g, beta, B, H, Dk, Dv, state, o, 0u, stream);
}

}  // extern "C"
