// kda_internal.h -- declarations shared by the library's translation units
// (host launchers implemented next to their kernels). Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Parameter-free front-end applied inside the kernels (KDA_FRONT_* of kda.h):
// q/k L2 normalisation with this epsilon inside the root, g read as u with
// log-decay -exp(u), beta read as a logit.
constexpr unsigned kFrontL2 = 1u, kFrontGate = 2u, kFrontBeta = 4u;
constexpr unsigned kFrontAll = kFrontL2 | kFrontGate | kFrontBeta;
constexpr float kL2Eps = 1e-6f;

// Attributes of the current device the launches depend on, queried once per
// device and process (later calls read the cached copy; hipGetDevice only).
// `valid` is false when the runtime could not be queried; the other fields
// then hold MI355X values.
struct DeviceInfo {
    bool valid = false;
    int cus = 256;                // compute units
    int lds_per_block = 65536;    // bytes of LDS one workgroup may use
    int lds_per_cu = 0;           // bytes of LDS per CU (0: unknown)
};
DeviceInfo device_info();

// ---- decode ---------------------------------------------------------------
hipError_t launch_decode(const void* q, const void* k, const void* v, bool bf16,
                         const float* g, const float* beta, int B, int H, int Dk, int Dv,
                         float* state, float* o, unsigned frontend, hipStream_t stream);

// ---- prefill --------------------------------------------------------------
// States requested at arbitrary positions: the positions of sequence s are
// values[offsets[s] .. offsets[s + 1]), each a token count P of that sequence
// (the state after its first P tokens goes to states[j, h]).
struct PosArgs {
    const int32_t* offsets = nullptr;  // [num_seqs + 1]; null: no positions
    const int32_t* values = nullptr;   // [num_pos]
    float* states = nullptr;           // [num_pos, H, Dk, Dv]
    int num_pos = 0;
};

// A second scan over the same chunks in the same launch as the first (the
// chunk-parallel path's scan of zero values from the identity): its values are
// one zero row read for every token and head (token and head strides 0); its
// initial and final states and its outputs have the first scan's shapes
// (Dk == Dv). Only the bf16 five-wave scan runs it.
struct TwinScan {
    const void* zero_v = nullptr;  // >= Dv zero values; null: no second scan
    const float* initial_state = nullptr;
    float* final_state = nullptr;
    float* o = nullptr;
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    bool bf16;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;  // may be null (one sequence)
    int num_seqs;
    int64_t total_tokens;
    int H, Dk, Dv;
    const float* initial_state;
    float* final_state;
    int64_t ckpt_interval;
    float* ckpt_states;
    int64_t ckpt_rows;
    float* o;
    void* workspace;
    size_t workspace_bytes;
    unsigned phases;    // bit 0: prepare (prep + K1), bit 1: scan (K2)
    unsigned frontend;  // kFront* bits (0: inputs used as given)
    PosArgs pos;
    TwinScan twin;      // scan phase only, no checkpoints or positions
    // varlen schedule tables (chunk_start, ckpt_base, order at the start of the
    // workspace) already written by the caller: the prepare phase skips prep
    bool schedule_ready = false;
};

// Bytes of workspace the plain prefill path needs (prep, K1, one scan).
size_t prefill_workspace_bytes(int64_t total_tokens, int num_seqs, int H, int Dk, int Dv,
                               bool bf16);

// The plain path: prep + K1 and/or one scan over all chunks of each sequence.
hipError_t launch_prefill_plain(const PrefillArgs& a, hipStream_t stream);

// Chunk-parallel path for one sequence with few heads (kda_split.hip):
// segments it would cut the sequence into on a device with `cus` CUs (1 = not
// used), and the workspace it needs when the workspace is sized for
// kSizingCUs (0 = never used for these sizes).
constexpr int kSizingCUs = 256;
int prefill_split_segments(int64_t total_tokens, int num_seqs, int H, int Dk, int Dv, bool bf16,
                           int cus);
size_t prefill_split_workspace_bytes(int64_t total_tokens, int num_seqs, int H, int Dk, int Dv,
                                     bool bf16);

// Whether a scan with a twin (TwinScan) in one launch beats two scans run one
// after the other, for npairs (sequence, head) pairs and Dv value columns.
bool prefill_twin_scan_pays(int npairs, int Dk, int Dv, bool bf16, int cus);

// Entry of every prefill call: the chunk-parallel path when it applies and the
// workspace allows it, else the plain path.
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Advances each stored chunk-start state of a requested position by the
// position's remaining P mod 64 tokens (implemented with the decode kernel).
hipError_t launch_advance(const PrefillArgs& a, hipStream_t stream);

// Upper bound on the number of 64-token chunks of a packed batch.
inline int64_t max_chunks(int64_t total_tokens, int num_seqs) {
    return total_tokens / 64 + num_seqs;
}

constexpr int kChunk = 64;

}  // namespace kda
