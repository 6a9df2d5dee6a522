// kda_prefill.hip -- chunked KDA prefill for gfx950: varlen prep, K1 (chunk
// tensor preparation) and K2 (blockwise recurrence over chunks).
//
// Algebra (derived from the token recurrence; the pages describe the two
// kernels in prose only: Kimi K3 report, "Methodology notes", FlashKDA
// bullet; SemiAnalysis digest, section 1, which names the UT transform).
// For one chunk of C = 64 rows starting from state S (Dk x Dv):
//   G      inclusive cumulative sum of g over the chunk's rows
//   A      = strictly-lower( diag(beta) (K*e^G)(K*e^-G)^T )         (C x C)
//   Ainv   = (I + A)^-1                       (unit lower-triangular)
//   W      = Ainv diag(beta) (K*e^G)          U0 = Ainv diag(beta) V
//   P      = lower-incl-diag( (Q*e^G)(K*e^-G)^T )
//   Qd     = Q*e^G,   Kc = K*e^(G_last - G),  Gamma_last = e^(G_last)
// and the chunk step of K2 is
//   U  = U0 - W S,    O = Qd S + P U,    S <- diag(Gamma_last) S + Kc^T U.
// K1 computes every S-independent quantity for all chunks in parallel and
// hands W, Qd, Kc^T, P, Ainv diag(beta) and Gamma_last to K2, which runs the
// sequential scan with S resident on chip.
//
// Numerics. The state S and every accumulation are fp32; A, its inverse and
// the decay exponents are fp32. With bf16 q/k/v the MFMA operands are fp16
// (one pass of v_mfma_f32_16x16x32_f16; fp16 keeps 11 significant bits, 8x
// finer than bf16, at the same matrix-core rate), and S enters W S and Qd S as
// an fp16 hi/lo pair. With fp32 q/k/v every product runs on
// v_mfma_f32_16x16x4_f32 with fp32 operands. Decay factors are formed as
// e^(G_r - G_ref) with a reference row per 16-row block, so the products
// never form e^(+G) of a whole chunk.
//
// Fragment convention (both operand types). A 16 x 32 (M x K) A-operand tile
// and a 32 x 16 (K x N) B-operand tile are held as 8 values per lane: lane l
// holds row (resp. column) l % 16 at K positions 8*(l/16) + e, e = 0..7.
// The f16 instruction consumes all 8 at once; the f32 path issues 8
// 16x16x4 instructions, instruction e consuming slot e. A 16 x 16 result tile
// gives lane l column l % 16, rows 4*(l/16) + i, i = 0..3. Within a 32-wide
// K slab, position 8q + e stands for index perm(q, e) = 4q + e (e < 4) or
// 16 + 4q + (e - 4) (e >= 4): then two stacked result tiles (rows 0-15 and
// 16-31 of a slab) ARE a B-operand fragment without any data movement, so
// S and U pass from accumulators to the next product as they are. Every
// handoff operand whose K index runs over channels or tokens of such a slab
// is stored with this permutation.
#include "kda_internal.h"

#include <type_traits>

namespace kda {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int C = kChunk;      // 64 tokens per chunk
constexpr int kThreads = 256;  // 4 waves
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
    return __uint_as_float(static_cast<unsigned>(b) << 16);
}

// K-slab permutation: slot (q, e) -> index inside a 32-wide slab.
__device__ __forceinline__ int perm32(int q, int e) {
    return e < 4 ? 4 * q + e : 16 + 4 * q + (e - 4);
}

// ---------------------------------------------------------------- MFMA ----
template <bool F16>
struct Mma;

template <>
struct Mma<true> {
    using E = _Float16;
    using Frag = half8;
    static __device__ __forceinline__ f32x4 run(const Frag& a, const Frag& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mma<false> {
    using E = float;
    using Frag = f32x8;
    static __device__ __forceinline__ f32x4 run(const Frag& a, const Frag& b, f32x4 c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
        return c;
    }
};

// Handoff block of one (head, chunk), in elements of E unless noted:
//   Wn  [4 row tiles][DK/32 slabs][64][8]   A-frags of -W   (rows tokens, K channels)
//   Qd  [4][DK/32][64][8]                   A-frags of Qd   (rows tokens, K channels)
//   KcT [DK/16 row tiles][2 slabs][64][8]   A-frags of Kc^T (rows channels, K tokens)
//   P   [4][2][64][8]                       A-frags of P    (rows tokens, K tokens)
//   Ab  [4][2][64][8]                       A-frags of Ainv diag(beta)
//   glast [DK] fp32                         Gamma_last
template <int DK, bool F16>
struct Handoff {
    using E = typename Mma<F16>::E;
    static constexpr int NKS = DK / 32;
    static constexpr int NRT = DK / 16;
    static constexpr size_t kW = 0;
    static constexpr size_t kQd = kW + 4 * NKS * 512;
    static constexpr size_t kKc = kQd + 4 * NKS * 512;
    static constexpr size_t kP = kKc + NRT * 2 * 512;
    static constexpr size_t kAb = kP + 4 * 2 * 512;
    static constexpr size_t kElems = kAb + 4 * 2 * 512;
    static constexpr size_t kGlastBytes = kElems * sizeof(E);
    static constexpr size_t kBytes = kGlastBytes + DK * sizeof(float);
    static_assert(kBytes % 256 == 0, "handoff block must keep 256-byte alignment");
};

size_t handoff_bytes(int Dk, bool bf16) {
    if (Dk == 64) return bf16 ? Handoff<64, true>::kBytes : Handoff<64, false>::kBytes;
    return bf16 ? Handoff<128, true>::kBytes : Handoff<128, false>::kBytes;
}

template <typename Frag, typename E>
__device__ __forceinline__ Frag load_frag(const E* base, int frag, int lane) {
    return *reinterpret_cast<const Frag*>(base + ((size_t)frag * 64 + lane) * 8);
}

template <typename Frag, typename E>
__device__ __forceinline__ void store_frag(E* base, int frag, int lane, const Frag& f) {
    *reinterpret_cast<Frag*>(base + ((size_t)frag * 64 + lane) * 8) = f;
}

// Workspace: [chunk_start: S+1][ckpt_base: S+1][order: S] int32, padded to
// 256 bytes, then the handoff blocks [H][max_chunks].
size_t table_bytes(int num_seqs) { return ((size_t)(3 * num_seqs + 2) * 4 + 255) / 256 * 256; }

// Token range [start, start + len) of sequence s, clamped to [0, N) so that a
// malformed cu_seqlens can never send an access out of bounds.
__device__ __forceinline__ void seq_range(const int32_t* cu, int s, int64_t N, int64_t& start,
                                          int64_t& len) {
    int64_t a = cu[s], b = cu[s + 1];
    a = a < 0 ? 0 : (a > N ? N : a);
    b = b < a ? a : (b > N ? N : b);
    start = a;
    len = b - a;
}

// ------------------------------------------------------------ varlen prep ----
// One workgroup: chunk_start = exclusive scan of ceil(L/64), ckpt_base =
// exclusive scan of floor(L/interval), order = sequences by decreasing length
// (ties by index) so that K2 starts the longest scans first.
__global__ __launch_bounds__(kThreads) void prep_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                        int64_t N, int64_t interval,
                                                        int32_t* __restrict__ chunk_start,
                                                        int32_t* __restrict__ ckpt_base,
                                                        int32_t* __restrict__ order) {
    __shared__ int32_t sc[kThreads], sk[kThreads];
    __shared__ int32_t carry_c, carry_k;
    const int t = threadIdx.x;
    if (t == 0) {
        carry_c = 0;
        carry_k = 0;
    }
    __syncthreads();
    for (int base = 0; base < num_seqs; base += kThreads) {
        const int s = base + t;
        int nc = 0, nk = 0;
        if (s < num_seqs) {
            int64_t st, L;
            seq_range(cu, s, N, st, L);
            nc = (int)((L + C - 1) / C);
            nk = interval > 0 ? (int)(L / interval) : 0;
        }
        sc[t] = nc;
        sk[t] = nk;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {  // inclusive Hillis-Steele scan
            const int a = t >= off ? sc[t - off] : 0;
            const int b = t >= off ? sk[t - off] : 0;
            __syncthreads();
            sc[t] += a;
            sk[t] += b;
            __syncthreads();
        }
        if (s < num_seqs) {
            chunk_start[s] = carry_c + sc[t] - nc;
            ckpt_base[s] = carry_k + sk[t] - nk;
        }
        __syncthreads();
        if (t == kThreads - 1) {
            carry_c += sc[t];
            carry_k += sk[t];
        }
        __syncthreads();
    }
    if (t == 0) {
        chunk_start[num_seqs] = carry_c;
        ckpt_base[num_seqs] = carry_k;
    }
    for (int s = t; s < num_seqs; s += kThreads) {
        int64_t st, L;
        seq_range(cu, s, N, st, L);
        int rank = 0;
        for (int r = 0; r < num_seqs; ++r) {
            int64_t str, Lr;
            seq_range(cu, r, N, str, Lr);
            rank += (Lr > L) || (Lr == L && r < s);
        }
        order[rank] = s;
    }
}

// Locate chunk ci: first token and length (len <= 0: no such chunk).
__device__ __forceinline__ void locate_chunk(int ci, const int32_t* cu, const int32_t* chunk_start,
                                             int num_seqs, int64_t N, int64_t& t0, int& len) {
    if (!cu) {
        t0 = (int64_t)ci * C;
        const int64_t rem = N - t0;
        len = rem <= 0 ? 0 : (rem < C ? (int)rem : C);
        return;
    }
    if (ci >= chunk_start[num_seqs]) {
        t0 = 0;
        len = 0;
        return;
    }
    int lo = 0, hi = num_seqs - 1;  // largest s with chunk_start[s] <= ci
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_start[mid] <= ci) lo = mid;
        else hi = mid - 1;
    }
    int64_t st, L;
    seq_range(cu, lo, N, st, L);
    const int64_t off = (int64_t)(ci - chunk_start[lo]) * C;
    t0 = st + off;
    const int64_t rem = L - off;
    len = rem <= 0 ? 0 : (rem < C ? (int)rem : C);
}

// ---------------------------------------------------------------- K1 -----
template <int DK, bool BF16>
__global__ __launch_bounds__(kThreads) void k1_prep_kernel(
    const void* __restrict__ qin, const void* __restrict__ kin, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_start, int num_seqs, int64_t N, int H, int64_t max_chunks,
    unsigned char* __restrict__ handoff) {
    using M = Mma<BF16>;
    using E = typename M::E;
    using Frag = typename M::Frag;
    using TIn = typename std::conditional<BF16, unsigned short, float>::type;
    using HO = Handoff<DK, BF16>;
    constexpr int NKS = DK / 32;
    constexpr int NRT = DK / 16;
    constexpr int VEC = 16 / sizeof(TIn);  // inputs per 16-byte load
    constexpr int KP = DK + VEC;           // padded LDS row of K
    constexpr int GP = DK + 4;             // padded LDS row of G
    constexpr int AP = C + 4;              // padded LDS row of A / Ainv
    constexpr int NQ = kThreads / DK;      // row groups of the cumulative sum
    constexpr int RPQ = C / NQ;

    __shared__ __attribute__((aligned(16))) TIn sK[C][KP];
    __shared__ __attribute__((aligned(16))) float sG[C][GP];  // G * log2(e)
    __shared__ __attribute__((aligned(16))) float sA[C][AP];  // A, then Ainv
    __shared__ float sB[C];
    __shared__ double sTot[NQ][DK];

    const int ci = blockIdx.x;
    const int h = blockIdx.y;
    int64_t t0;
    int len;
    locate_chunk(ci, cu, chunk_start, num_seqs, N, t0, len);
    if (len <= 0) return;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int q = lane >> 4;
    const int m = lane & 15;
    const TIn* K = static_cast<const TIn*>(kin);
    const TIn* Q = static_cast<const TIn*>(qin);
    E* hb = reinterpret_cast<E*>(handoff + ((size_t)h * max_chunks + ci) * HO::kBytes);
    float* glast = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(hb) + HO::kGlastBytes);

    auto row_off = [&](int r) -> int64_t { return ((t0 + r) * H + h) * (int64_t)DK; };

    // ---- stage K (zero rows past the chunk end), beta and the decay cumsum
    for (int i = t; i < C * DK / VEC; i += kThreads) {
        const int r = i / (DK / VEC);
        const int c = (i % (DK / VEC)) * VEC;
        typedef TIn vec_t __attribute__((ext_vector_type(VEC)));
        vec_t val = {};
        if (r < len) val = *reinterpret_cast<const vec_t*>(K + row_off(r) + c);
        *reinterpret_cast<vec_t*>(&sK[r][c]) = val;
    }
    if (t < C) sB[t] = t < len ? beta[(t0 + t) * H + h] : 0.f;
    {
        const int c = t % DK, grp = t / DK;
        double acc = 0.0;
        for (int r = grp * RPQ; r < (grp + 1) * RPQ; ++r)
            if (r < len) acc += (double)g[row_off(r) + c];
        sTot[grp][c] = acc;
        __syncthreads();
        double run = 0.0;
        for (int p = 0; p < grp; ++p) run += sTot[p][c];
        for (int r = grp * RPQ; r < (grp + 1) * RPQ; ++r) {
            if (r < len) run += (double)g[row_off(r) + c];
            sG[r][c] = (float)(run * 1.4426950408889634);
        }
    }
    __syncthreads();

    auto kval = [&](int r, int c) -> float {
        if constexpr (BF16) return bf16_to_f32(sK[r][c]);
        else return sK[r][c];
    };
    auto qval = [&](int r, int c) -> float {  // straight from global memory
        if (r >= len) return 0.f;
        if constexpr (BF16) return bf16_to_f32(Q[row_off(r) + c]);
        else return Q[row_off(r) + c];
    };

    // ---- phase A: A (strictly lower, into LDS) and P (handoff) per 16x16 block pair.
    // Block pair (rb, sb), sb <= rb, uses reference row 16*rb: every factor
    // e^(G_r - G_ref) (r >= ref) is <= 1 and e^(G_ref - G_s) is <= 1 for s < ref.
    {
        // pairs per wave, balanced: (rb, sb)
        const int pairs[4][3][2] = {{{3, 0}, {3, 1}, {0, 0}},
                                    {{3, 2}, {3, 3}, {1, 0}},
                                    {{2, 0}, {2, 1}, {-1, -1}},
                                    {{2, 2}, {1, 1}, {-1, -1}}};
        for (int pi = 0; pi < 3; ++pi) {
            const int rb = pairs[wave][pi][0], sb = pairs[wave][pi][1];
            if (rb < 0) break;
            const int ref = 16 * rb;
            const int r = 16 * rb + m;  // row of the X / Z operands
            const int s = 16 * sb + m;  // row of the Y operand
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                Frag X, Y, Z;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int c = 32 * ks + 8 * q + e;
                    const float gr = sG[r][c], gs = sG[s][c], gf = sG[ref][c];
                    const float fr = exp2f(gr - gf);
                    X[e] = (E)(kval(r, c) * fr);
                    Z[e] = (E)(qval(r, c) * fr);
                    Y[e] = (E)(kval(s, c) * exp2f(gf - gs));
                }
                accA = M::run(X, Y, accA);  // rows r, cols s
                accP = M::run(Y, Z, accP);  // P^T: rows s, cols r
            }
            // A[r'][s'] with r' = 16rb + 4q + i, s' = 16sb + m
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * rb + 4 * q + i, ss = 16 * sb + m;
                sA[rr][ss] = ss < rr ? sB[rr] * accA[i] : 0.f;
            }
            // P^T[s'][r'] with s' = 16sb + 4q + i, r' = 16rb + m -> P A-frag
            // [rt = rb][slab sb/2], slots 4*(sb%2) + i of lane (m + 16q).
            E* pf = hb + HO::kP + ((size_t)(rb * 2 + sb / 2) * 64 + lane) * 8 + 4 * (sb % 2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ss = 16 * sb + 4 * q + i, rr = 16 * rb + m;
                pf[i] = (E)(ss <= rr ? accP[i] : 0.f);
            }
        }
        // zero halves inside stored slabs: (rb, sb) = (0, 1) and (2, 3)
        if (wave == 2 || wave == 3) {
            const int rb = wave == 2 ? 0 : 2, sb = rb + 1;
            E* pf = hb + HO::kP + ((size_t)(rb * 2 + sb / 2) * 64 + lane) * 8 + 4 * (sb % 2);
#pragma unroll
            for (int i = 0; i < 4; ++i) pf[i] = (E)0.f;
        }
    }
    __syncthreads();

    // ---- phase B: wave 0 inverts (I + A) by forward substitution, lane j =
    // column j; the other waves write Qd, Kc^T and Gamma_last.
    if (wave == 0) {
        const int j = lane;
        float x[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int s4 = 0; s4 < r / 4 * 4; s4 += 4) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sA[r][s4]);
                acc -= a4[0] * x[s4] + a4[1] * x[s4 + 1] + a4[2] * x[s4 + 2] + a4[3] * x[s4 + 3];
            }
#pragma unroll
            for (int s = r / 4 * 4; s < r; ++s) acc -= sA[r][s] * x[s];
            x[r] = acc;
        }
        // all rows of A were consumed above: overwrite with Ainv (column j)
#pragma unroll
        for (int r = 0; r < C; ++r) sA[r][j] = x[r];
    } else {
        // Qd A-frags: rows tokens (tile rt), K channels (slab ks, permuted)
        for (int f = wave - 1; f < 4 * NKS; f += 3) {
            const int rt = f / NKS, ks = f % NKS;
            const int r = 16 * rt + m;
            Frag out;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 32 * ks + perm32(q, e);
                out[e] = (E)(qval(r, c) * exp2f(sG[r][c]));
            }
            store_frag<Frag, E>(hb + HO::kQd, rt * NKS + ks, lane, out);
        }
        // Kc^T A-frags: rows channels (tile ct), K tokens (slab ts, permuted)
        for (int f = wave - 1; f < NRT * 2; f += 3) {
            const int ct = f / 2, ts = f % 2;
            const int c = 16 * ct + m;
            const float gl = sG[C - 1][c];
            Frag out;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = 32 * ts + perm32(q, e);
                out[e] = (E)(kval(r, c) * exp2f(gl - sG[r][c]));
            }
            store_frag<Frag, E>(hb + HO::kKc, ct * 2 + ts, lane, out);
        }
        for (int c = t - 64; c < DK; c += kThreads - 64) glast[c] = exp2f(sG[C - 1][c]);
    }
    __syncthreads();

    // ---- phase C: -W from W^T = (diag(beta) Kd)^T Ainv^T and the Ab handoff.
    // W^T tiles (channel tile ct, token tile rt); tiles 2ks and 2ks+1 of the
    // same rt stack into the W A-frag of (rt, slab ks).
    for (int f = wave; f < 4 * NKS; f += 4) {
        const int ks = f % NKS, rt = f / NKS;
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        const int nts = rt >= 2 ? 2 : 1;  // Ainv[r][s] = 0 for s > r
        for (int ts = 0; ts < nts; ++ts) {
            Frag b;  // Ainv^T: column r = 16rt + m, K = s = 32ts + 8q + e
            const int r = 16 * rt + m;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = (E)sA[r][32 * ts + 8 * q + e];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                Frag a;  // (beta Kd)^T: row c = 16(2ks+half) + m, K = s
                const int c = 16 * (2 * ks + half) + m;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = 32 * ts + 8 * q + e;
                    a[e] = (E)(sB[s] * kval(s, c) * exp2f(sG[s][c]));
                }
                acc[half] = M::run(a, b, acc[half]);
            }
        }
        Frag out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[i] = (E)(-acc[0][i]);
            out[4 + i] = (E)(-acc[1][i]);
        }
        store_frag<Frag, E>(hb + HO::kW, rt * NKS + ks, lane, out);
    }
    // Ab = Ainv diag(beta) A-frags: rows tokens (tile rt), K tokens (slab ts, permuted);
    // slabs (rt 0-1, ts 1) are identically zero and never read.
    {
        const int frags[6][2] = {{0, 0}, {1, 0}, {2, 0}, {2, 1}, {3, 0}, {3, 1}};
        for (int f = wave; f < 6; f += 4) {
            const int rt = frags[f][0], ts = frags[f][1];
            const int r = 16 * rt + m;
            Frag out;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = 32 * ts + perm32(q, e);
                out[e] = (E)(sA[r][s] * sB[s]);
            }
            store_frag<Frag, E>(hb + HO::kAb, rt * 2 + ts, lane, out);
        }
    }
}

// ---------------------------------------------------------------- K2 -----
// One workgroup = one (sequence, head) and 16*NT value columns; wave w owns
// U/O row tile w (tokens 16w..16w+15) and state row tiles w*TPW .. +TPW-1.
template <int DK, int DV, int NT, bool BF16>
__global__ __launch_bounds__(kThreads) void k2_scan_kernel(
    const void* __restrict__ vin, const int32_t* __restrict__ cu, const int32_t* __restrict__ order,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ ckpt_base, int npairs,
    int64_t N, int H, int64_t max_chunks, const unsigned char* __restrict__ handoff,
    const float* __restrict__ s0, float* __restrict__ sfinal, int64_t interval,
    float* __restrict__ ckpt, int64_t ckpt_rows, float* __restrict__ o) {
    using M = Mma<BF16>;
    using E = typename M::E;
    using Frag = typename M::Frag;
    using TIn = typename std::conditional<BF16, unsigned short, float>::type;
    using HO = Handoff<DK, BF16>;
    constexpr int NKS = DK / 32;
    constexpr int TPW = DK / 64;            // state row tiles per wave
    constexpr int NVB = DV / (16 * NT);     // value-column blocks per (seq, head)
    constexpr int NV = 16 * NT;

    __shared__ __attribute__((aligned(32))) E sSh[NKS][NT][64][8];
    __shared__ __attribute__((aligned(32))) E sSl[BF16 ? NKS : 1][NT][64][8];
    __shared__ __attribute__((aligned(32))) E sV[2][NT][64][8];
    __shared__ __attribute__((aligned(32))) E sU[2][NT][64][8];

    // XCD-aware mapping: the NVB column blocks of one (seq, head) share an
    // XCD (workgroups are dealt to the 8 XCDs round-robin), so their common
    // handoff reads hit one L2.
    const int id = blockIdx.x;
    const int xcd = id & 7, slot = id >> 3;
    const int pair = xcd + 8 * (slot / NVB);
    const int vb = slot % NVB;
    if (pair >= npairs) return;
    const int rank = pair / H, h = pair % H;
    const int seq = order ? order[rank] : rank;
    int64_t tstart = 0, L = N;
    if (cu) seq_range(cu, seq, N, tstart, L);
    const int cbase = chunk_start ? chunk_start[seq] : 0;
    int nch = (int)((L + C - 1) / C);
    if (cbase + (int64_t)nch > max_chunks) nch = cbase < max_chunks ? (int)(max_chunks - cbase) : 0;
    const int j0 = vb * NV;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int q = lane >> 4;
    const int m = lane & 15;
    const TIn* V = static_cast<const TIn*>(vin);

    // state rows owned: channel 16*rt + 4q + i, column j0 + 16ct + m
    f32x4 S[TPW][NT];
    const size_t sbase = ((size_t)seq * H + h) * DK * DV;
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int row = 16 * (wave * TPW + i) + 4 * q + ii;
                S[i][ct][ii] = s0 ? s0[sbase + (size_t)row * DV + j0 + 16 * ct + m] : 0.f;
            }

    for (int n = 0; n < nch; ++n) {
        const E* hb = reinterpret_cast<const E*>(handoff + ((size_t)h * max_chunks + cbase + n) * HO::kBytes);
        const float* glast = reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(hb) + HO::kGlastBytes);
        const int64_t tok0 = tstart + (int64_t)n * C;
        const int len = (int)((L - (int64_t)n * C) < C ? (L - (int64_t)n * C) : C);

        // (a) publish S as B-frags (slab = row tile / 2, half = row tile % 2) and stage V
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int rt = wave * TPW + i;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                E* ph = &sSh[rt / 2][ct][lane][4 * (rt % 2)];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const E hi = (E)S[i][ct][ii];
                    ph[ii] = hi;
                    if constexpr (BF16) sSl[rt / 2][ct][lane][4 * (rt % 2) + ii] = (E)(S[i][ct][ii] - (float)hi);
                }
            }
        }
        for (int idx = t; idx < C * NV; idx += kThreads) {
            const int s = idx / NV, col = idx % NV;
            float val = 0.f;
            if (s < len) {
                const int64_t off = ((tok0 + s) * H + h) * (int64_t)DV + j0 + col;
                if constexpr (BF16) val = bf16_to_f32(V[off]);
                else val = V[off];
            }
            const int ts = s >> 5, w32 = s & 31;
            const int qq = (w32 & 15) >> 2;
            const int e = (w32 & 3) + ((w32 >> 4) << 2);
            sV[ts][col >> 4][(col & 15) + 16 * qq][e] = (E)val;
        }
        __syncthreads();

        // (c) U = Ab V - W S ; O = Qd S  (row tile = wave)
        const int rt = wave;
        const int nts = rt >= 2 ? 2 : 1;
        f32x4 U[NT], O[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            U[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            O[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int ts = 0; ts < nts; ++ts) {
            const Frag a = load_frag<Frag, E>(hb + HO::kAb, rt * 2 + ts, lane);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
                U[ct] = M::run(a, *reinterpret_cast<const Frag*>(&sV[ts][ct][lane][0]), U[ct]);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const Frag aw = load_frag<Frag, E>(hb + HO::kW, rt * NKS + ks, lane);
            const Frag aq = load_frag<Frag, E>(hb + HO::kQd, rt * NKS + ks, lane);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const Frag sh = *reinterpret_cast<const Frag*>(&sSh[ks][ct][lane][0]);
                U[ct] = M::run(aw, sh, U[ct]);
                O[ct] = M::run(aq, sh, O[ct]);
                if constexpr (BF16) {
                    const Frag sl = *reinterpret_cast<const Frag*>(&sSl[ks][ct][lane][0]);
                    U[ct] = M::run(aw, sl, U[ct]);
                    O[ct] = M::run(aq, sl, O[ct]);
                }
            }
        }
        // (d) publish U as B-frags (K = tokens): slab rt/2, half rt%2
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sU[rt / 2][ct][lane][4 * (rt % 2) + ii] = (E)U[ct][ii];
        __syncthreads();

        // (f) O += P U and store the valid rows
        for (int ts = 0; ts < nts; ++ts) {
            const Frag a = load_frag<Frag, E>(hb + HO::kP, rt * 2 + ts, lane);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
                O[ct] = M::run(a, *reinterpret_cast<const Frag*>(&sU[ts][ct][lane][0]), O[ct]);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int tok = 16 * rt + 4 * q + ii;
            if (tok < len) {
                float* op = o + ((tok0 + tok) * H + h) * (int64_t)DV + j0 + m;
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) op[16 * ct] = O[ct][ii];
            }
        }

        // (g) S <- diag(Gamma_last) S + Kc^T U
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int srt = wave * TPW + i;
            const f32x4 gl = *reinterpret_cast<const f32x4*>(glast + 16 * srt + 4 * q);
            const Frag a0 = load_frag<Frag, E>(hb + HO::kKc, srt * 2 + 0, lane);
            const Frag a1 = load_frag<Frag, E>(hb + HO::kKc, srt * 2 + 1, lane);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                f32x4 acc = S[i][ct] * gl;
                acc = M::run(a0, *reinterpret_cast<const Frag*>(&sU[0][ct][lane][0]), acc);
                acc = M::run(a1, *reinterpret_cast<const Frag*>(&sU[1][ct][lane][0]), acc);
                S[i][ct] = acc;
            }
        }

        // (h) checkpoint after every `interval` tokens of the sequence
        const int64_t done = (int64_t)(n + 1) * C;
        // (without cu_seqlens the only sequence has checkpoint base 0; rows the
        // caller's buffer does not have are skipped)
        const int64_t cidx = interval > 0 ? (int64_t)(ckpt_base ? ckpt_base[seq] : 0) + done / interval - 1 : -1;
        if (interval > 0 && done <= L && done % interval == 0 && cidx < ckpt_rows) {
            float* cp = ckpt + (cidx * H + h) * (size_t)DK * DV;
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const int row = 16 * (wave * TPW + i) + 4 * q + ii;
                        cp[(size_t)row * DV + j0 + 16 * ct + m] = S[i][ct][ii];
                    }
        }
    }

    if (sfinal) {
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int row = 16 * (wave * TPW + i) + 4 * q + ii;
                    sfinal[sbase + (size_t)row * DV + j0 + 16 * ct + m] = S[i][ct][ii];
                }
    }
}

// ------------------------------------------------------------- host side ---
struct Plan {
    int32_t* chunk_start;
    int32_t* ckpt_base;
    int32_t* order;
    unsigned char* handoff;
    int64_t max_chunks;
};

Plan make_plan(const PrefillArgs& a) {
    Plan p;
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    p.chunk_start = reinterpret_cast<int32_t*>(ws);
    p.ckpt_base = p.chunk_start + (a.num_seqs + 1);
    p.order = p.ckpt_base + (a.num_seqs + 1);
    p.handoff = ws + table_bytes(a.num_seqs);
    p.max_chunks = max_chunks(a.total_tokens, a.num_seqs);
    return p;
}

template <int DK, int DV, bool BF16>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
    const Plan p = make_plan(a);
    const bool varlen = a.cu_seqlens != nullptr;
    if (varlen)
        hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(kThreads), 0, stream, a.cu_seqlens, a.num_seqs,
                           a.total_tokens, a.ckpt_interval, p.chunk_start, p.ckpt_base, p.order);
    if (p.max_chunks > 0 && a.total_tokens > 0)
        hipLaunchKernelGGL((k1_prep_kernel<DK, BF16>), dim3((unsigned)p.max_chunks, (unsigned)a.H),
                           dim3(kThreads), 0, stream, a.q, a.k, a.g, a.beta, a.cu_seqlens,
                           varlen ? p.chunk_start : nullptr, a.num_seqs, a.total_tokens, a.H,
                           p.max_chunks, p.handoff);
    constexpr int NT = 1;
    constexpr int NVB = DV / (16 * NT);
    const int npairs = a.num_seqs * a.H;
    const int64_t groups = (npairs + 7) / 8;
    const unsigned grid = (unsigned)(groups * 8 * NVB);
    hipLaunchKernelGGL((k2_scan_kernel<DK, DV, NT, BF16>), dim3(grid), dim3(kThreads), 0, stream,
                       a.v, a.cu_seqlens, varlen ? p.order : nullptr,
                       varlen ? p.chunk_start : nullptr, varlen ? p.ckpt_base : nullptr, npairs,
                       a.total_tokens, a.H, p.max_chunks, p.handoff, a.initial_state, a.final_state,
                       a.ckpt_interval, a.ckpt_states, a.ckpt_rows, a.o);
    return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int64_t total_tokens, int num_seqs, int H, int Dk, int Dv,
                               bool bf16) {
    (void)Dv;
    return table_bytes(num_seqs) +
           (size_t)H * (size_t)max_chunks(total_tokens, num_seqs) * handoff_bytes(Dk, bf16);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    const bool b = a.bf16;
    if (a.Dk == 128 && a.Dv == 128) return b ? launch_typed<128, 128, true>(a, stream) : launch_typed<128, 128, false>(a, stream);
    if (a.Dk == 128 && a.Dv == 64) return b ? launch_typed<128, 64, true>(a, stream) : launch_typed<128, 64, false>(a, stream);
    if (a.Dk == 64 && a.Dv == 128) return b ? launch_typed<64, 128, true>(a, stream) : launch_typed<64, 128, false>(a, stream);
    if (a.Dk == 64 && a.Dv == 64) return b ? launch_typed<64, 64, true>(a, stream) : launch_typed<64, 64, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
