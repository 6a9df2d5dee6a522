// kda_split.hip -- chunk-parallel prefill of one sequence with few heads.
//
// The blockwise recurrence is sequential over chunks, so one sequence with
// few heads leaves most CUs idle: its scan has H * Dv / 16 column blocks. The
// chunk step is affine in the state (from the chunk algebra of the Kimi K3
// report's FlashKDA note, "Methodology notes"):
//     S_{n+1} = (Diag(Gamma_last) - Kc^T W) S_n + Kc^T U0,
// so a segment of chunks maps its start state X to M X + F, and every output
// row of the segment is o_t = o_t(X = 0) + (M_t^T q_t)^T X, where M_t is the
// product of the maps up to token t. The sequence is cut into P segments of
// whole chunks, treated as P independent pseudo-sequences:
//   1. prepare (K1) once for all segments, then scan A: the value columns with
//      the true initial state for segment 0 and zeros for the others
//      -> o(X = 0) into o, end states F_p;
//   2. scan B on the same handoff: zero values and the identity as initial
//      state -> end states M_p and outputs oI_t = (M_t^T q_t)^T, Dk columns;
//   3. combine (fp32, sequential over segments): scan A already started
//      segment 0 from S_0, so S_end(0) = F_0; for p >= 1 the true start state
//      is X_p = S_end(p-1) and S_end(p) = M_p X_p + F_p;
//   4. correct: o_t += oI_t X_p for every token of segments 1 .. P-1.
// Both scans run P * H * D / 16 column blocks at once over chains P times
// shorter; they are the plain path's kernels. With bf16 inputs and Dk == Dv
// they run in one launch of the five-wave scan when that pays: each of its
// workgroups shares one handoff stream among two column blocks (of one scan),
// the workgroups of both scans for a (segment, head) sit on one XCD and share
// its L2, and scan B reads one zero row for all its values instead of a zero
// tensor. The combine runs on fp32
// matrix cores and the correction at fp32 accuracy (three fp16 passes on
// hi/lo operand pairs scaled by powers of two, fp32 accumulation), for states
// of any magnitude.
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kT = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Upper limit on segments: keeps the sequential combine short.
constexpr int kMaxSegments = 16;
// Each segment spans at least this many chunks.
constexpr int64_t kMinSegmentChunks = 8;
// Fewer segments than this leave too little gain to pay for the second scan;
// with both scans in one launch (bf16, Dk == Dv) it costs less, and three pay
// (measured at T = 65536, D = 128: 1.13-1.17x at P = 3, 0.89-1.01x at P = 2).
constexpr int kMinSegments = 6;
constexpr int kMinSegmentsTwin = 3;

// Workspace of the split path, after the plain path's workspace for P
// pseudo-sequences (offsets in bytes, all 256-byte aligned).
struct SplitLayout {
    size_t plain, pcu, init_a, fin_a, xst, init_b, fin_b, zero_v, o_i, end;
};

SplitLayout split_layout(int64_t N, int P, int H, int Dk, int Dv, bool bf16) {
    SplitLayout L;
    const size_t st_v = (size_t)P * H * Dk * Dv * sizeof(float);
    const size_t st_k = (size_t)P * H * Dk * Dk * sizeof(float);
    L.plain = align256(prefill_workspace_bytes(N, P, H, Dk, Dv, bf16));
    L.pcu = L.plain;
    L.init_a = L.pcu + align256((size_t)(P + 1) * sizeof(int32_t));
    L.fin_a = L.init_a + align256(st_v);
    L.xst = L.fin_a + align256(st_v);
    L.init_b = L.xst + align256(st_v);
    L.fin_b = L.init_b + align256(st_k);
    L.zero_v = L.fin_b + align256(st_k);
    L.o_i = L.zero_v + align256((size_t)N * H * Dk * (bf16 ? 2 : 4));
    L.end = L.o_i + align256((size_t)N * H * Dk * sizeof(float));
    return L;
}

// ---------------------------------------------------------------- fill ----
// Pseudo-sequence boundaries and their schedule tables (what the varlen prep
// would compute: every segment but the last has seg_chunks chunks, none has
// checkpoints, and longest first is index order), scan A's initial states
// (segment 0: the caller's, else zeros), scan B's identity initial states,
// zero values.
__global__ __launch_bounds__(kT) void split_fill_kernel(int32_t* __restrict__ pcu,
                                                        int32_t* __restrict__ tables, int P,
                                                        int64_t seg_tokens, int64_t N,
                                                        const float* __restrict__ s0,
                                                        float* __restrict__ init_a,
                                                        float* __restrict__ init_b,
                                                        f32x4* __restrict__ zero_v, int64_t zero_vec4,
                                                        int H, int Dk, int Dv) {
    const int64_t tid = (int64_t)blockIdx.x * kT + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kT;
    if (tid <= P) {
        const int64_t b = tid * seg_tokens;
        pcu[tid] = (int32_t)(b < N ? b : N);
        // chunk_start [P + 1], ckpt_base [P + 1], order [P]
        const int64_t nchunks = (N + 63) / 64, c = tid * (seg_tokens / 64);
        tables[tid] = (int32_t)(c < nchunks ? c : nchunks);
        tables[P + 1 + tid] = 0;
        if (tid < P) tables[2 * (P + 1) + tid] = (int32_t)tid;
    }
    const int64_t one = (int64_t)H * Dk * Dv;  // states of one pseudo-sequence
    for (int64_t i = tid; i < (int64_t)P * one; i += stride)
        init_a[i] = (i < one && s0 != nullptr) ? s0[i] : 0.f;
    const int64_t sq = (int64_t)Dk * Dk;
    for (int64_t i = tid; i < (int64_t)P * H * sq; i += stride) {
        const int64_t e = i % sq;
        init_b[i] = (e / Dk == e % Dk) ? 1.f : 0.f;
    }
    for (int64_t i = tid; i < zero_vec4; i += stride) zero_v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ------------------------------------------------------------- combine ----
// One workgroup per (head, 16 value columns), sequential over segments:
//   S_end(0) = F_0;  for p >= 1: X_p = S_end(p-1), S_end(p) = M_p X_p + F_p.
// X_p (p >= 1) goes to xst for the output correction; S_end(P-1) is the final
// state. M_p X_p runs on v_mfma_f32_16x16x4_f32 with one wave per 16-row tile
// of the state (DK / 16 waves). K step (s, e) takes K index 16 s + 4 g + e in
// lane group g, so each lane reads 16-byte pieces of its M row; X (K x 16
// columns) sits in LDS. M and F do not depend on the chain: each wave loads
// them two segments ahead.
template <int DK, int P>
__global__ __launch_bounds__(DK * 4) void split_combine_kernel(const float* __restrict__ fin_a,
                                                               const float* __restrict__ fin_b,
                                                               float* __restrict__ xst,
                                                               float* __restrict__ final_state,
                                                               int H, int Dv) {
    constexpr int NT = DK * 4;   // threads
    constexpr int KS = DK / 16;  // 16-byte pieces per M row
    constexpr int XP = DK + 4;   // padded LDS row of X^T
    // X_p^T for every segment (column c of the block is row c here, so a
    // lane's four K values of a K step are one 16-byte read and its four
    // result rows one 16-byte write). Slot p holds X_p (slot P: the final
    // state); the chain stores nothing to global memory until it is done,
    // so its waits on the operand loads never wait for stores as well.
    __shared__ __attribute__((aligned(16))) float sXs[P + 1][16][XP];
    const int h = blockIdx.x, j0 = blockIdx.y * 16;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m = lane & 15, q = lane >> 4;
    const size_t sv = (size_t)DK * Dv, sk = (size_t)DK * DK;
    struct Step {
        f32x4 A[KS];
        f32x4 F;
    };
    auto load_step = [&](int p, Step& st) {
        if (p >= P) return;
        const float* M = fin_b + ((size_t)p * H + h) * sk + (size_t)(16 * wave + m) * DK + 4 * q;
        const float* Fp = fin_a + ((size_t)p * H + h) * sv + (size_t)(16 * wave + 4 * q) * Dv + j0 + m;
#pragma unroll
        for (int s = 0; s < KS; ++s) st.A[s] = *reinterpret_cast<const f32x4*>(M + 16 * s);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.F[i] = Fp[(size_t)i * Dv];
    };
    // X_1 = S_end(0) = F_0 (all loads issued before the first LDS write)
    constexpr int PER = DK * 16 / NT;  // state elements per thread
    {
        float x1[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = t + NT * k;
            x1[k] = fin_a[((size_t)h * DK + i / 16) * Dv + j0 + i % 16];
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = t + NT * k;
            sXs[1][i % 16][i / 16] = x1[k];
        }
    }
    // Step p uses buffer p % NB; the loads for step p + NB - 1 go into the
    // buffer step p - 1 has finished with. The segment count is a template
    // parameter and the loop fully unrolled: every buffer index is a constant
    // and, with no loop back-edge or guard, each wait covers exactly the loads
    // its step needs (a back-edge or a join would wait for every load).
    constexpr int NB = 4;  // operand buffers: loads run NB - 1 steps ahead
    Step buf[NB];
#pragma unroll
    for (int p = 1; p < NB; ++p) load_step(p, buf[p % NB]);
    __syncthreads();
#pragma unroll
    for (int p = 1; p < P; ++p) {
        load_step(p + NB - 1, buf[(p + NB - 1) % NB]);
        const Step& cur = buf[p % NB];
        f32x4 b[KS];  // X_p[16 s + 4 q + e][m]
#pragma unroll
        for (int s = 0; s < KS; ++s) b[s] = *reinterpret_cast<const f32x4*>(&sXs[p][m][16 * s + 4 * q]);
        // four independent accumulation chains (K steps e = 0..3), summed at the end
        f32x4 acc[4] = {cur.F, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.A[s][e], b[s][e], acc[e], 0, 0, 0);
        // S_end(p) = X_{p+1}: rows 16 wave + 4 q + i, column m
        *reinterpret_cast<f32x4*>(&sXs[p + 1][m][16 * wave + 4 * q]) = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        __syncthreads();
    }
    // X_p (p = 1 .. P-1) for the output correction, X_P = S_end(P-1) is the final state
#pragma unroll
    for (int p = 1; p <= P; ++p) {
        float* dst = p < P ? xst + ((size_t)p * H + h) * sv : final_state;
        if (p == P) {
            if (final_state == nullptr) break;
            dst += (size_t)h * sv;
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = t + NT * k;
            dst[(size_t)(i / 16) * Dv + j0 + i % 16] = sXs[p][i % 16][i / 16];
        }
    }
}

// ------------------------------------------------ split fp16 products ----
// The output correction runs its fp32 product on the fp16 matrix cores with
// each operand split into a pair x = hi + lo of fp16 values and three passes of
// v_mfma_f32_16x16x32_f16 (hi hi, hi lo, lo hi) accumulated in fp32: the
// dropped lo lo term is about 2^-22 of each product, so the result keeps fp32
// accuracy at three times the fp16 rate instead of the fp32 matrix-core rate
// (8x lower). Each wave scales its operand by a power of two (exact) so that
// its largest magnitude lies in [2^14, 2^15): every hi and lo then fits fp16,
// whatever the magnitudes of the states, and the result is scaled back.
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// Exponent k such that the wave's largest |x| (amax, this lane's share)
// times 2^k lies in [2^14, 2^15); 0 when every value is zero.
__device__ __forceinline__ int wave_scale_exp(float amax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    return amax > 0.f ? 15 - __builtin_amdgcn_frexp_expf(amax) : 0;
}

// x * 2^k split into fp16 hi and lo
struct HalfPair {
    _Float16 hi, lo;
};
__device__ __forceinline__ HalfPair split_pair(float x, int k) {
    const float xs = ldexpf(x, k);
    const _Float16 hi = (_Float16)xs;
    return HalfPair{hi, (_Float16)(xs - (float)hi)};
}

__device__ __forceinline__ float abs_max4(float a, f32x4 v) {
    return fmaxf(fmaxf(a, fmaxf(fabsf(v[0]), fabsf(v[1]))), fmaxf(fabsf(v[2]), fabsf(v[3])));
}

// ---------------------------------------------------------- correction ----
// o_t += oI_t X_p for the tokens of segments 1 .. P-1, as the transposed
// product (o_corr)^T = X_p^T oI^T (a split fp16 product, above), so that each
// lane's result is four consecutive value columns of one token (16-byte
// read-modify-write of o). One workgroup per (head, segment, kGroup
// chunks inside the segment); wave w owns value-column tiles w + 4 j, whose
// X_p^T operand pairs stay in registers. Each 16-token tile of oI is loaded
// once per workgroup (every thread a share, one tile ahead) into a
// double-buffered LDS tile that all four waves read their operands from;
// each wave loads the old o values of its own columns one tile ahead.
// (Measured at T = 65536, H = 4, P = 8: 103 us with every wave loading the
// whole oI tile itself, 83 us shared through LDS; 94 us with four chunks per
// workgroup, 121 us loading two tiles ahead.)
// Fragments: lane l holds row (A) or column (B) l % 16 at K = 8 (l / 16) + e.
constexpr int kGroup = 2;  // chunks per workgroup

template <int DK, int DV>
__global__ __launch_bounds__(kT) void split_correct_kernel(const float* __restrict__ o_i,
                                                           const float* __restrict__ xst,
                                                           float* __restrict__ o, int64_t N, int H,
                                                           int64_t seg_chunks, int64_t groups_per_seg) {
    constexpr int CTW = DV / 64;  // column tiles per wave
    constexpr int KS = DK / 32;   // 32-wide K steps
    constexpr int NTILE = kGroup * 4;
    constexpr int BP = DK + 4;           // padded LDS row of the oI tile
    constexpr int NV = 16 * DK / 4 / kT;  // 16-byte oI pieces per thread and tile
    static_assert(NV >= 1 && 16 * DK / 4 == NV * kT, "oI tile pieces spread evenly over the threads");
    __shared__ __attribute__((aligned(16))) float sB[2][16][BP];
    const int h = (int)(blockIdx.x % (unsigned)H);
    const int64_t wg = (int64_t)(blockIdx.x / (unsigned)H);
    const int p = 1 + (int)(wg / groups_per_seg);
    const int64_t c0 = p * seg_chunks + (wg % groups_per_seg) * kGroup;
    // tokens of this workgroup that belong to segment p and exist
    int64_t t_end = (p + 1) * seg_chunks * 64;
    t_end = t_end < N ? t_end : N;
    const int64_t t_begin = c0 * 64;
    if (t_begin >= t_end) return;  // uniform over the workgroup
    int64_t t_stop = t_begin + 64 * kGroup;
    t_stop = t_stop < t_end ? t_stop : t_end;  // this workgroup's tokens: [t_begin, t_stop)
    const int ntile = (int)((t_stop - t_begin + 15) / 16);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m = lane & 15, q = lane >> 4;
    // A = X_p^T: row 16 ct + m, K = 32 ks + 8 q + e, scaled by 2^ka
    half8 ahi[CTW][KS], alo[CTW][KS];
    int ka;
    {
        const float* X = xst + ((size_t)p * H + h) * DK * DV;
        float xa[CTW][KS][8];
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < CTW; ++j)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xa[j][ks][e] = X[(size_t)(32 * ks + 8 * q + e) * DV + 16 * (wave + 4 * j) + m];
                    am = fmaxf(am, fabsf(xa[j][ks][e]));
                }
        ka = wave_scale_exp(am);
#pragma unroll
        for (int j = 0; j < CTW; ++j)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const HalfPair hp = split_pair(xa[j][ks][e], ka);
                    ahi[j][ks][e] = hp.hi;
                    alo[j][ks][e] = hp.lo;
                }
    }
    // rows outside [t_begin, t_stop) are read from t_begin (in bounds) and not stored
    auto row_at = [&](int64_t tok) { return (tok < t_stop ? tok : t_begin) * H + h; };
    f32x4 stage[NV];  // this thread's share of the next oI tile
    auto load_stage = [&](int u) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = t + kT * i, r = v / (DK / 4), c = v % (DK / 4);
            stage[i] = *reinterpret_cast<const f32x4*>(o_i + row_at(t_begin + 16 * u + r) * (int64_t)DK + 4 * c);
        }
    };
    auto put_stage = [&](int b) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = t + kT * i, r = v / (DK / 4), c = v % (DK / 4);
            *reinterpret_cast<f32x4*>(&sB[b][r][4 * c]) = stage[i];
        }
    };
    f32x4 old[2][CTW];  // old o of this wave's columns, token m of the tile
    auto load_old = [&](int u, f32x4* dst) {
        const float* src = o + row_at(t_begin + 16 * u + m) * (int64_t)DV + 4 * q;
#pragma unroll
        for (int j = 0; j < CTW; ++j) dst[j] = *reinterpret_cast<const f32x4*>(src + 16 * (wave + 4 * j));
    };
    load_stage(0);
    load_old(0, old[0]);
#pragma unroll
    for (int u = 0; u < NTILE; ++u) {
        if (u >= ntile) break;  // uniform
        put_stage(u & 1);
        if (u + 1 < ntile) {
            load_stage(u + 1);
            load_old(u + 1, old[(u + 1) & 1]);
        }
        __syncthreads();  // tile u in LDS; every wave is done with tile u - 1
        half8 bhi[KS], blo[KS];  // B = oI^T: column = token m, K = 32 ks + 8 q + e, scaled by 2^kb
        f32x4 vb[2 * KS];
        float bm = 0.f;
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) {
            vb[i] = *reinterpret_cast<const f32x4*>(&sB[u & 1][m][32 * (i >> 1) + 8 * q + 4 * (i & 1)]);
            bm = abs_max4(bm, vb[i]);
        }
        const int kb = wave_scale_exp(bm);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const HalfPair hp = split_pair(vb[2 * ks + (e >> 2)][e & 3], kb);
                bhi[ks][e] = hp.hi;
                blo[ks][e] = hp.lo;
            }
        f32x4 acc[CTW][2];
#pragma unroll
        for (int j = 0; j < CTW; ++j) {
            acc[j][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < CTW; ++j) {
                acc[j][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[j][ks], bhi[ks], acc[j][0], 0, 0, 0);
                acc[j][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[j][ks], blo[ks], acc[j][1], 0, 0, 0);
                acc[j][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[j][ks], bhi[ks], acc[j][1], 0, 0, 0);
            }
        const int64_t tok = t_begin + 16 * u + m;
        if (tok < t_stop) {
            float* dst = o + (tok * H + h) * (int64_t)DV + 4 * q;
#pragma unroll
            for (int j = 0; j < CTW; ++j) {
                const f32x4 r = acc[j][0] + acc[j][1];
                f32x4 out;
#pragma unroll
                for (int i = 0; i < 4; ++i) out[i] = old[u & 1][j][i] + ldexpf(r[i], -(ka + kb));
                *reinterpret_cast<f32x4*>(dst + 16 * (wave + 4 * j)) = out;
            }
        }
    }
}

template <int DK, int DV>
hipError_t launch_fix(const float* fin_a, const float* fin_b, float* xst, float* final_state,
                      const float* o_i, float* o, int64_t N, int H, int P, int64_t seg_chunks,
                      hipStream_t stream) {
    const dim3 grid((unsigned)H, DV / 16), block(DK * 4);
    switch (P) {
#define KDA_COMBINE(NP)                                                                        \
    case NP:                                                                                   \
        hipLaunchKernelGGL((split_combine_kernel<DK, NP>), grid, block, 0, stream, fin_a, fin_b, \
                           xst, final_state, H, DV);                                           \
        break;
        KDA_COMBINE(3) KDA_COMBINE(4) KDA_COMBINE(5) KDA_COMBINE(6) KDA_COMBINE(7) KDA_COMBINE(8) KDA_COMBINE(9)
        KDA_COMBINE(10)
        KDA_COMBINE(11) KDA_COMBINE(12) KDA_COMBINE(13) KDA_COMBINE(14) KDA_COMBINE(15)
        KDA_COMBINE(16)
#undef KDA_COMBINE
        default: return hipErrorInvalidValue;
    }
    const int64_t groups_per_seg = (seg_chunks + kGroup - 1) / kGroup;
    const int64_t wgs = (int64_t)(P - 1) * groups_per_seg * H;
    if (wgs > 0)
        hipLaunchKernelGGL((split_correct_kernel<DK, DV>), dim3((unsigned)wgs), dim3(kT), 0, stream,
                           o_i, xst, o, N, H, seg_chunks, groups_per_seg);
    return hipGetLastError();
}

}  // namespace

int prefill_split_segments(int64_t total_tokens, int num_seqs, int H, int Dk, int Dv, bool bf16,
                           int cus) {
    if (num_seqs != 1 || total_tokens <= 0 || cus <= 0) return 1;
    const int64_t nchunks = (total_tokens + 63) / 64;
    const int64_t blocks = (int64_t)H * ((Dk > Dv ? Dk : Dv) / 16);  // wider scan's workgroups
    int64_t P = cus / blocks;
    P = P < nchunks / kMinSegmentChunks ? P : nchunks / kMinSegmentChunks;
    P = P < kMaxSegments ? P : kMaxSegments;
    // two scans of 1/P of the chain plus the combine and the correction: measured
    // on MI355X (D = 128, T = 65536) with two scan launches 3.3x faster than the
    // plain scan at P = 16, 1.7x at P = 8, 1.05x at P = 4
    if (P < (bf16 && Dk == Dv ? kMinSegmentsTwin : kMinSegments)) return 1;
    const int64_t seg = (nchunks + P - 1) / P;
    return (int)((nchunks + seg - 1) / seg);
}

size_t prefill_split_workspace_bytes(int64_t total_tokens, int num_seqs, int H, int Dk, int Dv,
                                     bool bf16) {
    const int P = prefill_split_segments(total_tokens, num_seqs, H, Dk, Dv, bf16, kSizingCUs);
    if (P < 2) return 0;
    return split_layout(total_tokens, P, H, Dk, Dv, bf16).end;
}

hipError_t launch_fix_dims(const float* fin_a, const float* fin_b, float* xst, const PrefillArgs& a,
                           const float* o_i, int64_t N, int P, int64_t seg_chunks, hipStream_t stream) {
    if (a.Dk == 128 && a.Dv == 128) return launch_fix<128, 128>(fin_a, fin_b, xst, a.final_state, o_i, a.o, N, a.H, P, seg_chunks, stream);
    if (a.Dk == 128 && a.Dv == 64) return launch_fix<128, 64>(fin_a, fin_b, xst, a.final_state, o_i, a.o, N, a.H, P, seg_chunks, stream);
    if (a.Dk == 64 && a.Dv == 128) return launch_fix<64, 128>(fin_a, fin_b, xst, a.final_state, o_i, a.o, N, a.H, P, seg_chunks, stream);
    if (a.Dk == 64 && a.Dv == 64) return launch_fix<64, 64>(fin_a, fin_b, xst, a.final_state, o_i, a.o, N, a.H, P, seg_chunks, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    const bool eligible = a.cu_seqlens == nullptr && a.num_seqs == 1 && a.phases == 3u &&
                          a.ckpt_interval == 0 && a.pos.num_pos == 0 && a.total_tokens > 0;
    int P = 1;
    if (eligible) {
        const DeviceInfo di = device_info();
        if (di.valid) {
            const int cus = di.cus;
            const int want = prefill_split_segments(a.total_tokens, 1, a.H, a.Dk, a.Dv, a.bf16, cus);
            const int sized = prefill_split_segments(a.total_tokens, 1, a.H, a.Dk, a.Dv, a.bf16, kSizingCUs);
            // the workspace was sized for `sized` segments: never use more
            P = want < sized ? want : sized;
            if (P >= 2 && split_layout(a.total_tokens, P, a.H, a.Dk, a.Dv, a.bf16).end > a.workspace_bytes)
                P = 1;
        }
    }
    if (P < 2) return launch_prefill_plain(a, stream);

    const int64_t N = a.total_tokens;
    const int64_t nchunks = (N + 63) / 64;
    const int64_t seg_chunks = (nchunks + P - 1) / P;
    const SplitLayout L = split_layout(N, P, a.H, a.Dk, a.Dv, a.bf16);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    int32_t* pcu = reinterpret_cast<int32_t*>(ws + L.pcu);
    float* init_a = reinterpret_cast<float*>(ws + L.init_a);
    float* fin_a = reinterpret_cast<float*>(ws + L.fin_a);
    float* xst = reinterpret_cast<float*>(ws + L.xst);
    float* init_b = reinterpret_cast<float*>(ws + L.init_b);
    float* fin_b = reinterpret_cast<float*>(ws + L.fin_b);
    void* zero_v = ws + L.zero_v;
    float* o_i = reinterpret_cast<float*>(ws + L.o_i);

    // Both scans in one launch when that pays (bf16, Dk == Dv): the second
    // reads one zero row for every token; else a zero value tensor.
    const DeviceInfo di = device_info();
    const bool twin = prefill_twin_scan_pays(P * a.H, a.Dk, a.Dv, a.bf16, di.cus);
    const int64_t zero_vec4 = twin ? a.Dk * 2 / 16 : N * a.H * a.Dk * (a.bf16 ? 2 : 4) / 16;
    {
        const int64_t work = (int64_t)P * a.H * a.Dk * (a.Dk > a.Dv ? a.Dk : a.Dv);
        const int64_t most = work > zero_vec4 ? work : zero_vec4;
        int64_t blocks = (most + kT - 1) / kT;
        blocks = blocks < 4096 ? blocks : 4096;
        hipLaunchKernelGGL(split_fill_kernel, dim3((unsigned)blocks), dim3(kT), 0, stream, pcu,
                           static_cast<int32_t*>(a.workspace), P, seg_chunks * 64, N, a.initial_state, init_a, init_b,
                           static_cast<f32x4*>(zero_v), zero_vec4, a.H, a.Dk, a.Dv);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    PrefillArgs A = a;  // scan A: value columns, end states F_p, outputs o(X = 0)
    A.cu_seqlens = pcu;
    A.num_seqs = P;
    A.initial_state = init_a;
    A.final_state = fin_a;
    A.workspace_bytes = L.plain;
    A.schedule_ready = true;  // written by the fill
    hipError_t e;
    if (twin) {
        A.phases = 1u;  // prep + K1
        e = launch_prefill_plain(A, stream);
        if (e != hipSuccess) return e;
        A.phases = 2u;  // scans A and B in one launch
        A.twin.zero_v = zero_v;
        A.twin.initial_state = init_b;
        A.twin.final_state = fin_b;
        A.twin.o = o_i;
        e = launch_prefill_plain(A, stream);
        if (e != hipSuccess) return e;
        return launch_fix_dims(fin_a, fin_b, xst, a, o_i, N, P, seg_chunks, stream);
    }
    e = launch_prefill_plain(A, stream);
    if (e != hipSuccess) return e;
    PrefillArgs Bs = A;  // scan B: zero values from the identity -> M_p, oI
    Bs.v = zero_v;
    Bs.Dv = a.Dk;
    Bs.initial_state = init_b;
    Bs.final_state = fin_b;
    Bs.o = o_i;
    Bs.phases = 2u;
    e = launch_prefill_plain(Bs, stream);
    if (e != hipSuccess) return e;
    return launch_fix_dims(fin_a, fin_b, xst, a, o_i, N, P, seg_chunks, stream);
}

}  // namespace kda
