// kda_decode.hip -- single-token KDA decode step for gfx950.
//
// Per (batch row b, head h) the step is
//     a = exp(g);  S' = Diag(a) S;  r = S'^T k;  p = S'^T q
//     u = beta (v - r);  o = p + (k . q) u;  S <- S' + k u^T
// which is S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T and
// o = S_t^T q written so that every state element is read once and written
// once. The pages size this step at about 7*D^2 FLOPs against 8*D^2 bytes of
// fp32 state traffic per head and token (Kimi K3 report, "Key data"): under
// one FLOP per byte, so the kernel is built for HBM bandwidth, with no MFMA.
//
// Mapping: one 512-thread workgroup per (b, h) (for batches that do not give
// every CU 8 of them, 2 or 4 workgroups per (b, h), each owning a slice of
// the value columns: decode_slices_kernel). Thread t owns the 4 adjacent
// value columns 4*(t % CG) .. +3 (CG = Dv/4) of the key rows
// rg, rg + RG, rg + 2*RG, ... (rg = t / CG, RG = 512/CG): one wave reads
// 64/CG whole adjacent rows per 16-byte-per-lane load, so each load
// instruction moves 1 KiB of contiguous state. The decayed slab stays in
// VGPRs between the reduction and the write-back; r, p and k.q are reduced
// across row groups with lane shuffles and then across the 8 waves in LDS, in
// a fixed order (bitwise reproducible).
//
// Residency: HBM sustains this read-then-write stream best with few state
// blocks in flight per CU. Measured on MI355X for 64 KiB states
// (B = 512, H = 32, D = 128): one 512-thread workgroup per CU moves
// 6.1-6.2 TB/s; two per CU 5.8; the default residency (four) 5.4; 256-thread
// workgroups 5.4-5.55 at any residency. The launch therefore asks for enough
// (unused) dynamic LDS that only n workgroups fit on a CU, n = 64 KiB / state
// bytes (at least 1), keeping about 64 KiB of state in flight per CU.
//
// Optional parameter-free front-end (KDA's query/key L2 normalisation and
// gate activations; Kimi K3 report, "Methodology notes", Kimi Delta
// Attention): with L2, k and q are scaled by 1/sqrt(sum x^2 + 1e-6) in fp32
// (every wave loads both rows and reduces their norms itself while the state
// is in flight; the butterfly gives every lane the same bits); `front` bit kFrontGate reads g as u and uses -exp(u), bit
// kFrontBeta reads beta as a logit and uses its sigmoid.
#include "kda_internal.h"

#include <type_traits>

namespace kda {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
    return __uint_as_float(static_cast<unsigned>(b) << 16);
}

template <bool BF16>
__device__ __forceinline__ float load_in(const void* p, int64_t i) {
    if constexpr (BF16)
        return bf16_to_f32(static_cast<const unsigned short*>(p)[i]);
    else
        return static_cast<const float*>(p)[i];
}

// Raw input element (bf16 bits or fp32), converted later by in_f32: keeps the
// wait for the load out of the code that issues the next loads.
template <bool BF16>
using raw_t = typename std::conditional<BF16, unsigned short, float>::type;

template <bool BF16>
__device__ __forceinline__ raw_t<BF16> load_raw(const void* p, int64_t i) {
    return static_cast<const raw_t<BF16>*>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ float in_f32(raw_t<BF16> x) {
    if constexpr (BF16) return bf16_to_f32(x);
    else return x;
}

template <bool BF16>
__device__ __forceinline__ f32x4 load_in4(const void* p, int64_t i) {
    if constexpr (BF16) {
        u16x4 b = *reinterpret_cast<const u16x4*>(static_cast<const unsigned short*>(p) + i);
        return f32x4{bf16_to_f32(b.x), bf16_to_f32(b.y), bf16_to_f32(b.z), bf16_to_f32(b.w)};
    } else {
        return *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
    }
}

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

template <int DK, int DV, bool BF16, bool L2>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    float* __restrict__ o, unsigned front) {
    constexpr int CG = DV / 4;           // column groups (threads per row)
    constexpr int RG = kThreads / CG;    // row groups
    constexpr int RPT = DK / RG;         // rows per thread
    constexpr int RGW = 64 / CG;         // row groups per wave
    static_assert(RPT * RG == DK && CG * 4 == DV && RGW >= 1, "bad decode tiling");

    // per-row vectors, one slot per thread: every thread stores its slot (rows
    // past DK are never read), so no branch invites the compiler to sink the
    // row loads behind the state loads
    __shared__ float s_a[kThreads], s_k[kThreads], s_q[kThreads];
    __shared__ f32x4 s_red[kWaves][CG][2];
    __shared__ float s_kq[kWaves];

    const int t = threadIdx.x;
    const int cg = t % CG;
    const int rg = t / CG;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int64_t pair = blockIdx.x;  // b * H + h
    float* S = state + pair * (int64_t)(DK * DV);

    // 1. the small per-(b, h) inputs first: the memory counter completes in
    // issue order, so waiting for them does not wait for the state
    static_assert(DK <= kThreads, "one key row per thread");
    const int tr = t < DK ? t : DK - 1;  // unconditional loads (no branch to join)
    float graw = g[pair * DK + tr];
    const raw_t<BF16> kraw = load_raw<BF16>(k, pair * DK + tr);
    const raw_t<BF16> qraw = load_raw<BF16>(q, pair * DK + tr);
    const f32x4 vv = load_in4<BF16>(v, pair * DV + 4 * cg);
    float bt = beta[pair];
    raw_t<BF16> kw[L2 ? DK / 64 : 1], qw[L2 ? DK / 64 : 1];  // whole k and q rows for the norms
    if constexpr (L2) {
#pragma unroll
        for (int j = 0; j < DK / 64; ++j) {
            kw[j] = load_raw<BF16>(k, pair * DK + lane + 64 * j);
            qw[j] = load_raw<BF16>(q, pair * DK + lane + 64 * j);
        }
    }
    asm volatile("" ::: "memory");  // keep them ahead of the state loads
    __builtin_amdgcn_sched_barrier(0);

    // 2. stream the thread's state slab in (all loads in flight at once)
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(S + (int64_t)(rg + m * RG) * DV) + cg);
    __builtin_amdgcn_sched_barrier(0);

    // while the state is in flight: activations, norms, per-row vectors to LDS
    if (front & kFrontGate) graw = -__expf(graw);
    s_a[t] = __expf(graw);
    s_k[t] = in_f32<BF16>(kraw);
    s_q[t] = in_f32<BF16>(qraw);
    if (front & kFrontBeta) bt = 1.f / (1.f + __expf(-bt));
    float kn = 1.f, qn = 1.f;  // inverse norms of k and q (L2)
    if constexpr (L2) {
        // No contraction here: a lane's last square fused into the first
        // exchange's addition would be unrounded in that lane only, and the
        // lanes (so the row groups) would get different norms.
#pragma clang fp contract(off)
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < DK / 64; ++j) {
            const float kx = in_f32<BF16>(kw[j]), qx = in_f32<BF16>(qw[j]);
            sk = j == 0 ? kx * kx : fmaf(kx, kx, sk);
            sq = j == 0 ? qx * qx : fmaf(qx, qx, sq);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            sk += __shfl_xor(sk, off);
            sq += __shfl_xor(sq, off);
        }
        kn = 1.f / sqrtf(sk + kL2Eps);
        qn = 1.f / sqrtf(sq + kL2Eps);
    }
    __syncthreads();

    // 3. decay in registers; partial S'^T k, S'^T q and k.q over this thread's rows
    f32x4 r = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        const float ai = s_a[i], ki = s_k[i] * kn, qi = s_q[i] * qn;
        s[m] *= ai;
        r += s[m] * ki;
        p += s[m] * qi;
        kq += ki * qi;
    }

    // 4. reduce over the row groups of this wave (lanes CG apart)
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] += __shfl_xor(r[e], off);
            p[e] += __shfl_xor(p[e], off);
        }
        kq += __shfl_xor(kq, off);
    }
    if (lane < CG) {
        s_red[wave][lane][0] = r;
        s_red[wave][lane][1] = p;
    }
    if (lane == 0) s_kq[wave] = kq;
    __syncthreads();

    // 5. across waves (fixed order), then the delta-rule correction u
    f32x4 rr = s_red[0][cg][0], pp = s_red[0][cg][1];
    float kqt = s_kq[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        rr += s_red[w][cg][0];
        pp += s_red[w][cg][1];
        kqt += s_kq[w];
    }
    // (every key row belongs to exactly one row group, so kqt = k . q)
    const f32x4 u = bt * (vv - rr);
    if (rg == 0) {
        const f32x4 out = pp + kqt * u;
        *reinterpret_cast<f32x4*>(o + pair * DV + 4 * cg) = out;
    }

    // 6. rank-1 write and stream the slab back out
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        const f32x4 nv = s[m] + (s_k[i] * kn) * u;
        __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + (int64_t)i * DV) + cg);
    }
}

// Column slices (few (b, h) pairs): the step of decode_kernel with NS
// workgroups of 512 / NS threads per (b, h), slice j owning value columns
// j DV/NS .. (j+1) DV/NS - 1 (every step of the update is per value column,
// except k . q, which each slice forms itself). A thread keeps the tiling of
// decode_kernel (rows rg, rg + RG, ... for RG = 2048 / DV row groups; 4
// adjacent columns), and the reductions over row groups run in the same
// order: a butterfly over each run of RGW = 256 / DV consecutive row groups
// (one wave's worth in decode_kernel), then the RG / RGW run sums in
// ascending order. So a (b, h) gets the same bits whatever its batch's size.
template <int DK, int DV, int NS, bool BF16, bool L2>
__global__ __launch_bounds__(kThreads / NS) void decode_slices_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    float* __restrict__ o, unsigned front) {
    constexpr int NT = kThreads / NS;    // threads of this workgroup
    constexpr int CG = DV / 4;           // column groups of the whole state
    constexpr int CGS = CG / NS;         // column groups of this slice
    constexpr int RG = kThreads / CG;    // row groups
    constexpr int RPT = DK / RG;         // rows per thread
    constexpr int RGW = 64 / CG;         // row groups per run (a wave at NS = 1)
    constexpr int NRUN = RG / RGW;       // runs
    static_assert(RPT * RG == DK && CG * 4 == DV && RGW >= 1 && CGS * NS == CG && CGS >= 1 &&
                      NT % 64 == 0 && NRUN == kWaves,
                  "bad decode tiling");

    // per-row vectors: every thread stores its slots (rows past DK are never
    // read), so no branch invites the compiler to sink the row loads behind
    // the state loads
    constexpr int RPS = (DK + NT - 1) / NT;  // per-row slots per thread
    __shared__ float s_a[RPS * NT], s_k[RPS * NT], s_q[RPS * NT];
    __shared__ f32x4 s_red[NRUN][CGS][2];
    __shared__ float s_kq[NRUN];

    const int t = threadIdx.x;
    const int cgl = t % CGS;  // column group within the slice
    const int rg = t / CGS;
    const int lane = t & 63;
    const int64_t pair = blockIdx.x / NS;  // b * H + h
    const int cg = (int)(blockIdx.x % NS) * CGS + cgl;
    float* S = state + pair * (int64_t)(DK * DV);

    // 1. the small per-(b, h) inputs first: the memory counter completes in
    // issue order, so waiting for them does not wait for the state
    float graw[RPS];
    raw_t<BF16> kraw[RPS], qraw[RPS];
#pragma unroll
    for (int j = 0; j < RPS; ++j) {
        const int i = t + NT * j;
        const int tr = i < DK ? i : DK - 1;  // unconditional loads (no branch to join)
        graw[j] = g[pair * DK + tr];
        kraw[j] = load_raw<BF16>(k, pair * DK + tr);
        qraw[j] = load_raw<BF16>(q, pair * DK + tr);
    }
    const f32x4 vv = load_in4<BF16>(v, pair * DV + 4 * cg);
    float bt = beta[pair];
    raw_t<BF16> kw[L2 ? DK / 64 : 1], qw[L2 ? DK / 64 : 1];  // whole k and q rows for the norms
    if constexpr (L2) {
#pragma unroll
        for (int j = 0; j < DK / 64; ++j) {
            kw[j] = load_raw<BF16>(k, pair * DK + lane + 64 * j);
            qw[j] = load_raw<BF16>(q, pair * DK + lane + 64 * j);
        }
    }
    asm volatile("" ::: "memory");  // keep them ahead of the state loads
    __builtin_amdgcn_sched_barrier(0);

    // 2. stream the thread's state slab in (all loads in flight at once)
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(S + (int64_t)(rg + m * RG) * DV) + cg);
    __builtin_amdgcn_sched_barrier(0);

    // while the state is in flight: activations, norms, per-row vectors to LDS
#pragma unroll
    for (int j = 0; j < RPS; ++j) {
        float gj = graw[j];
        if (front & kFrontGate) gj = -__expf(gj);
        s_a[t + NT * j] = __expf(gj);
        s_k[t + NT * j] = in_f32<BF16>(kraw[j]);
        s_q[t + NT * j] = in_f32<BF16>(qraw[j]);
    }
    if (front & kFrontBeta) bt = 1.f / (1.f + __expf(-bt));
    float kn = 1.f, qn = 1.f;  // inverse norms of k and q (L2)
    if constexpr (L2) {
        // No contraction here: a lane's last square fused into the first
        // exchange's addition would be unrounded in that lane only, and the
        // lanes (so the row groups and slices) would get different norms.
#pragma clang fp contract(off)
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < DK / 64; ++j) {
            const float kx = in_f32<BF16>(kw[j]), qx = in_f32<BF16>(qw[j]);
            sk = j == 0 ? kx * kx : fmaf(kx, kx, sk);
            sq = j == 0 ? qx * qx : fmaf(qx, qx, sq);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            sk += __shfl_xor(sk, off);
            sq += __shfl_xor(sq, off);
        }
        kn = 1.f / sqrtf(sk + kL2Eps);
        qn = 1.f / sqrtf(sq + kL2Eps);
    }
    __syncthreads();

    // 3. decay in registers; partial S'^T k, S'^T q and k.q over this thread's rows
    f32x4 r = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        const float ai = s_a[i], ki = s_k[i] * kn, qi = s_q[i] * qn;
        s[m] *= ai;
        r += s[m] * ki;
        p += s[m] * qi;
        kq += ki * qi;
    }

    // 4. butterfly over each run of RGW row groups (lanes CGS apart)
#pragma unroll
    for (int j = 1; j < RGW; j <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] += __shfl_xor(r[e], CGS * j);
            p[e] += __shfl_xor(p[e], CGS * j);
        }
        kq += __shfl_xor(kq, CGS * j);
    }
    if (rg % RGW == 0) {
        s_red[rg / RGW][cgl][0] = r;
        s_red[rg / RGW][cgl][1] = p;
        if (cgl == 0) s_kq[rg / RGW] = kq;
    }
    __syncthreads();

    // 5. run sums in ascending order, then the delta-rule correction u
    f32x4 rr = s_red[0][cgl][0], pp = s_red[0][cgl][1];
    float kqt = s_kq[0];
#pragma unroll
    for (int w = 1; w < NRUN; ++w) {
        rr += s_red[w][cgl][0];
        pp += s_red[w][cgl][1];
        kqt += s_kq[w];
    }
    // (every key row belongs to exactly one row group, so kqt = k . q)
    const f32x4 u = bt * (vv - rr);
    if (rg == 0) {
        const f32x4 out = pp + kqt * u;
        *reinterpret_cast<f32x4*>(o + pair * DV + 4 * cg) = out;
    }

    // 6. rank-1 write and stream the slab back out
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        const f32x4 nv = s[m] + (s_k[i] * kn) * u;
        __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + (int64_t)i * DV) + cg);
    }
}

// Dynamic LDS (never touched by the kernel) that leaves room for only
// n = max(1, 64 KiB / slice state bytes) decode workgroups per CU: each asks
// for lds_per_cu / (n + 1/2) bytes in all, more than a share of n + 1 and no
// more than a share of n.
template <int DK, int DV, int NS>
unsigned residency_pad() {
    constexpr int NT = kThreads / NS, CGS = DV / 4 / NS;
    constexpr int RPS = (DK + NT - 1) / NT;
    constexpr int kStatic = 3 * RPS * NT * 4 + kWaves * CGS * 2 * 16 + kWaves * 4;
    constexpr int kSlice = DK * DV * 4 / NS;
    const int n = (kSlice >= 65536) ? 1 : 65536 / kSlice;
    const DeviceInfo di = device_info();
    if (!di.valid || di.lds_per_cu <= 0) return 0;
    const int lds = di.lds_per_cu, per_block = di.lds_per_block;
    const int64_t want = (int64_t)lds * 2 / (2 * n + 1) - kStatic;
    if (want <= 0 || want + kStatic > per_block) return 0;  // cannot pad: default residency
    return (unsigned)want;
}

template <int DK, int DV, int NS>
hipError_t launch_slices(const void* q, const void* k, const void* v, bool bf16, const float* g,
                         const float* beta, int B, int H, float* state, float* o, unsigned front,
                         hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)B * H * NS)), block(kThreads / NS);
    const unsigned pad = residency_pad<DK, DV, NS>();
    const bool l2 = (front & kFrontL2) != 0;
    void (*kern)(const void*, const void*, const void*, const float*, const float*, float*, float*, unsigned);
    if constexpr (NS == 1)
        kern = bf16 ? (l2 ? &decode_kernel<DK, DV, true, true> : &decode_kernel<DK, DV, true, false>)
                    : (l2 ? &decode_kernel<DK, DV, false, true> : &decode_kernel<DK, DV, false, false>);
    else
        kern = bf16 ? (l2 ? &decode_slices_kernel<DK, DV, NS, true, true> : &decode_slices_kernel<DK, DV, NS, true, false>)
                    : (l2 ? &decode_slices_kernel<DK, DV, NS, false, true> : &decode_slices_kernel<DK, DV, NS, false, false>);
    hipLaunchKernelGGL(kern, grid, block, pad, stream, q, k, v, g, beta, state, o, front);
    return hipGetLastError();
}

// Slices per (b, h), from kernel-trace times on MI355X (D = 128, bf16,
// H = 32, 256 CUs), with 1 / 2 / 4 slices: B = 1: 4.24 / 3.68 / 3.48 us;
// B = 4: 5.36 / 4.72 / 4.68; B = 8: 6.48 / 5.64 / 5.64; B = 32: 24.7 / 23.2 /
// 23.5; B = 64: 47.8 / 46.1 / 47.3; B = 128: 90.4 / 90.8 / 93.5; B = 512:
// 350 / 380 / 383. So four slices while the pairs cover at most half the
// CUs, two up to 8 pairs per CU, else one.
template <int DK, int DV>
hipError_t launch_dims(const void* q, const void* k, const void* v, bool bf16, const float* g,
                       const float* beta, int B, int H, float* state, float* o, unsigned front,
                       hipStream_t stream) {
    const int64_t pairs = (int64_t)B * H;
    const int64_t cus = device_info().cus;
    if (2 * pairs <= cus) return launch_slices<DK, DV, 4>(q, k, v, bf16, g, beta, B, H, state, o, front, stream);
    if (pairs <= 8 * cus) return launch_slices<DK, DV, 2>(q, k, v, bf16, g, beta, B, H, state, o, front, stream);
    return launch_slices<DK, DV, 1>(q, k, v, bf16, g, beta, B, H, state, o, front, stream);
}

// ------------------------------------------------- position advance ----
// Sum over the 16 lanes of a DPP row, left in every lane of the row: two
// quad permutations, then rotations by 4 and 8 within the row (VALU lane
// moves, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp_mov<0x124>(x);  // row_ror:4
    x += dpp_mov<0x128>(x);  // row_ror:8
    return x;
}

// States at arbitrary positions (kda_prefill_chunked_at): for a position of
// P tokens the scan stored the state at the start of the chunk that holds P;
// this kernel runs the remaining r = P mod 64 tokens of the recurrence on it,
// in place (no outputs), one workgroup per (position, head), with the state
// in registers. The same front-end bits apply as in the prefill that produced
// the chunk-start state.
template <int DK, int DV, bool BF16, bool L2>
__global__ __launch_bounds__(kThreads) void advance_kernel(
    const void* __restrict__ kin, const void* __restrict__ vin, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu, int num_seqs, int64_t N,
    int H, PosArgs pos, unsigned front) {
    // One workgroup per (position, head). Wave w owns value columns
    // w * CPW .. +CPW-1 (every key row); lane = 16 * cgl + rgl holds the four
    // columns of group cgl for the rows rgl + 16 m, so the reduction S'^T k
    // over rows is one 16-lane DPP row sum and the token loop has no barrier.
    constexpr int CPW = DV / kWaves;  // columns per wave (16 or 8)
    constexpr int CGW = CPW / 4;      // 4-column groups per wave (4 or 2)
    constexpr int RPL = DK / 16;      // rows per lane (8 or 4)
    static_assert(CGW * 4 == CPW && RPL * 16 == DK && CGW * 16 <= 64, "bad advance tiling");

    // the (at most 63) rows the position still needs, staged once: their loads
    // are all in flight together instead of one token's worth per step
    __shared__ __attribute__((aligned(16))) float s_g[63][DK], s_k[63][DK], s_v[63][DV];  // s_g: alpha
    __shared__ float s_b[64];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int cgl = lane >> 4, rgl = lane & 15;
    const bool active = cgl < CGW;  // DV = 64: lanes 32..63 mirror 0..31 and store nothing
    const int col = wave * CPW + 4 * (active ? cgl : 0);
    const int j = (int)(blockIdx.x / (unsigned)H), h = (int)(blockIdx.x % (unsigned)H);

    // sequence of position j: the last s with offsets[s] <= j (clamped ranges)
    int64_t st = 0, L = N;
    if (cu) {
        int lo = 0, hi = num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pos.offsets[mid] <= j) lo = mid;
            else hi = mid - 1;
        }
        int64_t a = cu[lo], b = cu[lo + 1];
        a = a < 0 ? 0 : (a > N ? N : a);
        b = b < a ? a : (b > N ? N : b);
        st = a;
        L = b - a;
    }
    int64_t P = pos.values[j];
    P = P < 0 ? 0 : (P > L ? L : P);
    const int r = (int)(P % 64);
    if (r == 0) return;  // the scan stored the exact state
    const int64_t t0 = st + (P - r);
    float* S = pos.states + ((size_t)j * H + h) * (size_t)(DK * DV);

    f32x4 s[RPL];
#pragma unroll
    for (int m = 0; m < RPL; ++m)
        s[m] = *reinterpret_cast<const f32x4*>(S + (int64_t)(rgl + 16 * m) * DV + col);
    // every staging load in flight at once: 4-element vectors, at most
    // ceil(63 * D / 4 / 512) = 4 of each tensor per thread
    constexpr int NVK = (63 * DK / 4 + kThreads - 1) / kThreads;
    constexpr int NVV = (63 * DV / 4 + kThreads - 1) / kThreads;
    f32x4 gv[NVK], kv[NVK], vv[NVV];
#pragma unroll
    for (int u = 0; u < NVK; ++u) {
        const int idx = t + u * kThreads;  // (row, 4-channel group)
        const int i = idx / (DK / 4), c = 4 * (idx % (DK / 4));
        const int64_t e = ((t0 + i) * H + h) * DK + c;
        if (i < r) {
            gv[u] = *reinterpret_cast<const f32x4*>(g + e);
            kv[u] = load_in4<BF16>(kin, e);
        }
    }
#pragma unroll
    for (int u = 0; u < NVV; ++u) {
        const int idx = t + u * kThreads;
        const int i = idx / (DV / 4), c = 4 * (idx % (DV / 4));
        if (i < r) vv[u] = load_in4<BF16>(vin, ((t0 + i) * H + h) * DV + c);
    }
    float bt = t < r ? beta[(t0 + t) * H + h] : 0.f;
#pragma unroll
    for (int u = 0; u < NVK; ++u) {
        const int idx = t + u * kThreads;
        const int i = idx / (DK / 4), c = 4 * (idx % (DK / 4));
        if (i < r) {
            // decay factors alpha = e^g, formed here for all rows at once
            // instead of on the token chain
            f32x4 gi = gv[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (front & kFrontGate) gi[e] = -__expf(gi[e]);
                gi[e] = __expf(gi[e]);
            }
            *reinterpret_cast<f32x4*>(&s_g[i][c]) = gi;
            *reinterpret_cast<f32x4*>(&s_k[i][c]) = kv[u];
        }
    }
#pragma unroll
    for (int u = 0; u < NVV; ++u) {
        const int idx = t + u * kThreads;
        const int i = idx / (DV / 4), c = 4 * (idx % (DV / 4));
        if (i < r) *reinterpret_cast<f32x4*>(&s_v[i][c]) = vv[u];
    }
    if (t < r) {
        if (front & kFrontBeta) bt = 1.f / (1.f + __expf(-bt));
        s_b[t] = bt;
    }
    __syncthreads();  // the only barrier: everything below reads LDS only

    // token loop; each token's LDS operands are read one token ahead
    float gn[RPL], kn_[RPL];
    f32x4 vn;
    float bn;
    auto fetch = [&](int i) {
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            gn[m] = s_g[i][rgl + 16 * m];
            kn_[m] = s_k[i][rgl + 16 * m];
        }
        vn = *reinterpret_cast<const f32x4*>(&s_v[i][col]);
        bn = s_b[i];
    };
    fetch(0);
    for (int i = 0; i < r; ++i) {
        float gc[RPL], kc[RPL];
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            gc[m] = gn[m];
            kc[m] = kn_[m];
        }
        const f32x4 vc = vn;
        const float bc = bn;
        fetch(i + 1 < r ? i + 1 : i);
        if constexpr (L2) {  // key norm over the 16 row groups (every lane: same bits)
            float sk = 0.f;
#pragma unroll
            for (int m = 0; m < RPL; ++m) sk += kc[m] * kc[m];
            const float inv = 1.f / sqrtf(row_sum16(sk) + kL2Eps);
#pragma unroll
            for (int m = 0; m < RPL; ++m) kc[m] *= inv;
        }
        // decay, then S'^T k over the lane's rows and the DPP row's 16 row groups
        f32x4 rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            s[m] *= gc[m];
            rr += s[m] * kc[m];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[e] = row_sum16(rr[e]);
        const f32x4 u = bc * (vc - rr);
#pragma unroll
        for (int m = 0; m < RPL; ++m) s[m] += kc[m] * u;
    }
    if (active) {
#pragma unroll
        for (int m = 0; m < RPL; ++m)
            *reinterpret_cast<f32x4*>(S + (int64_t)(rgl + 16 * m) * DV + col) = s[m];
    }
}

template <int DK, int DV>
hipError_t launch_advance_dims(const PrefillArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)a.pos.num_pos * a.H)), block(kThreads);
    const bool l2 = (a.frontend & kFrontL2) != 0;
    auto kern = a.bf16 ? (l2 ? &advance_kernel<DK, DV, true, true> : &advance_kernel<DK, DV, true, false>)
                       : (l2 ? &advance_kernel<DK, DV, false, true> : &advance_kernel<DK, DV, false, false>);
    hipLaunchKernelGGL(kern, grid, block, 0, stream, a.k, a.v, a.g, a.beta, a.cu_seqlens,
                       a.num_seqs, a.total_tokens, a.H, a.pos, a.frontend);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, bool bf16,
                         const float* g, const float* beta, int B, int H, int Dk, int Dv,
                         float* state, float* o, unsigned front, hipStream_t stream) {
    if ((int64_t)B * H == 0) return hipSuccess;
    if (Dk == 128 && Dv == 128) return launch_dims<128, 128>(q, k, v, bf16, g, beta, B, H, state, o, front, stream);
    if (Dk == 128 && Dv == 64) return launch_dims<128, 64>(q, k, v, bf16, g, beta, B, H, state, o, front, stream);
    if (Dk == 64 && Dv == 128) return launch_dims<64, 128>(q, k, v, bf16, g, beta, B, H, state, o, front, stream);
    if (Dk == 64 && Dv == 64) return launch_dims<64, 64>(q, k, v, bf16, g, beta, B, H, state, o, front, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda

namespace kda {

hipError_t launch_advance(const PrefillArgs& a, hipStream_t stream) {
    if (a.pos.num_pos <= 0 || a.H <= 0) return hipSuccess;
    if (a.Dk == 128 && a.Dv == 128) return launch_advance_dims<128, 128>(a, stream);
    if (a.Dk == 128 && a.Dv == 64) return launch_advance_dims<128, 64>(a, stream);
    if (a.Dk == 64 && a.Dv == 128) return launch_advance_dims<64, 128>(a, stream);
    if (a.Dk == 64 && a.Dv == 64) return launch_advance_dims<64, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
