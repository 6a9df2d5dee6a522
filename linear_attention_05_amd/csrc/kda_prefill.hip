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
// finer than bf16, at the same matrix-core rate), S and U entering their
// products rounded to fp16 once. With fp32 q/k/v every product runs on
// v_mfma_f32_16x16x4_f32 with fp32 operands.
//
// Decay range. Every decay factor an operand carries is e^(G_a - G_b) with
// a >= b, i.e. at most 1, so no operand overflows for any g <= 0 and a factor
// that underflows is off by less than the operand type's smallest step. A
// pair (r, s) of rows in different 16-row blocks splits at the first row of
// r's block (both halves <= 1). Inside a diagonal 16-row block the split
// row must lie between s and r, which no single reference does for all
// pairs; when the decay summed over the block is small in every channel
// (below 2^12 for fp16 operands) the block still uses its first row (factors
// in [2^-12, 2^12]: fp16 keeps full precision). Otherwise the channels that
// decay more than that over the block, when there are at most 16 of them,
// are left out of its products and their pairs summed exactly in fp32 on the
// vector units (each pair's factor 2^-|G_r - G_s| formed on its own); with
// more, the block is done as four products, one per bit of the 16-row
// index: at level h the rows with bit h set take e^(G_r - G_{start of r's
// h-run}) and the rows with bit h clear take e^(G_{start of the next h-run}
// - G_s), and each product keeps only the pairs whose highest differing
// index bit is h. The per-token
// log-decay is floored at -kGFloor nats (alpha >= e^-16 for bf16 inputs,
// e^-64 for fp32: the change it makes to any result is below 1e-7 of the
// state), which keeps |G| over a chunk small enough that differences of the
// stored G (fp32 for bf16 inputs, fp64 for fp32 inputs, from an fp64
// cumulative sum) lose at most 1.2e-4 of a factor's log2, below the fp16
// operand rounding.
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
#include <utility>

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
// per-token log-decay floor (nats), by input type (see "Decay range" above)
constexpr float kGFloorBF16 = 16.f, kGFloorF32 = 64.f;
// a diagonal 16-row block keeps one reference row while the decay summed
// over it stays below this many powers of two in every channel
constexpr float kSpanLog2BF16 = 12.f, kSpanLog2F32 = 60.f;
// a diagonal block with at most this many channels over the span sums those
// channels' pairs on the vector units and the rest with one reference row;
// with more it takes the four-level products
constexpr int kSlowChannelsVALU = 16;


__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
    return __uint_as_float(static_cast<unsigned>(b) << 16);
}

// An input element (bf16 bits or fp32) as fp32.
template <typename T>
__device__ __forceinline__ float qf_in(T v) {
    if constexpr (std::is_same<T, float>::value) return v;
    else return bf16_to_f32(v);
}

// Sum of a value over lane pairs (l, l ^ 16) / (l, l ^ 32), with the two
// addends in the same order in both lanes (v_permlane16/32_swap).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float pair_sum16(float v) {
    const u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum32(float v) {
    const u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x on the hardware exponential (inputs here are differences of decay
// sums, far from the range where the library wrapper's rescaling matters).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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
    // P and Ab are lower triangular over the chunk's tokens: of their
    // (row tile, token slab) frags only the six that hold entries are stored,
    // (0,0) (1,0) (2,0) (2,1) (3,0) (3,1) in that order
    static constexpr size_t kAb = kP + 6 * 512;
    static constexpr size_t kElems = kAb + 6 * 512;
    static __host__ __device__ constexpr int tri(int rt, int ts) { return rt < 2 ? rt : 2 * rt - 2 + ts; }
    static constexpr size_t kGlastBytes = kElems * sizeof(E);
    static constexpr size_t kBytes = kGlastBytes + DK * sizeof(float);
    static_assert(kBytes % 256 == 0, "handoff block must keep 256-byte alignment");
};

size_t handoff_bytes(int Dk, bool bf16) {
    if (Dk == 64) return bf16 ? Handoff<64, true>::kBytes : Handoff<64, false>::kBytes;
    return bf16 ? Handoff<128, true>::kBytes : Handoff<128, false>::kBytes;
}

// f(std::integral_constant<int, k>) for k = 0 .. N-1, each k a constant
template <typename F, int... Ks>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Ks...>) {
    (f(std::integral_constant<int, Ks>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
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
// 256 bytes, a sink for stores the scan issues without a branch but does not
// need (512 KiB: 64 workgroup slots x 256 threads x 8 floats), then the handoff
// blocks [H][max_chunks].
constexpr int kSinkSlots = 64;     // workgroup slots (power of two)
constexpr int kSinkFloats = 8;     // floats per thread and slot
constexpr size_t kSinkBytes = (size_t)kSinkSlots * kThreads * kSinkFloats * sizeof(float);
size_t table_bytes(int num_seqs) { return ((size_t)(3 * num_seqs + 2) * 4 + 255) / 256 * 256 + kSinkBytes; }

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
// One workgroup of 1024 threads; two passes over the sequences in tiles of
// 8192 (8 consecutive sequences per thread), O(num_seqs) work:
//   pass 1  chunk_start = exclusive scan of ceil(L/64) and ckpt_base =
//           exclusive scan of floor(L/interval) (thread sums, wave scans, then
//           the 16 wave totals), and a histogram of the sequences' length
//           classes (half octaves of the chunk count)
//   pass 2  order = sequences by decreasing length class, ties by index, so
//           that K2 starts the longest scans first: a stable counting sort,
//           ranks among equal classes within a wave from lane ballots and
//           across waves and tiles from per-class counters.
constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / 64;
constexpr int kPrepPer = 8;                              // sequences per thread and tile
constexpr int kPrepTile = kPrepThreads * kPrepPer;
constexpr int kClasses = 64;

// Length class of a sequence of nc chunks: nc itself below 4, then two
// classes per octave (nc < 2^26 gives at most 51). Non-decreasing in nc.
__device__ __forceinline__ int length_class(int nc) {
    if (nc < 4) return nc;
    const int e = 31 - __clz(nc);
    return 2 * e + ((nc >> (e - 1)) & 1);
}

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                            int64_t N, int64_t interval,
                                                            int32_t* __restrict__ chunk_start,
                                                            int32_t* __restrict__ ckpt_base,
                                                            int32_t* __restrict__ order) {
    __shared__ int sWsum[2][kPrepWaves];          // per-wave totals of a tile
    __shared__ int sHist[kClasses];               // sequences per class
    __shared__ int sBase[kClasses];               // next order slot of each class
    __shared__ int sWcnt[kPrepWaves][kClasses];   // pass 2: per-wave class counts
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    auto chunks_of = [&](int s, int64_t& L) {
        int64_t st;
        seq_range(cu, s, N, st, L);
        return (int)((L + C - 1) / C);
    };
    for (int i = t; i < kClasses; i += kPrepThreads) sHist[i] = 0;
    for (int i = t; i < kPrepWaves * kClasses; i += kPrepThreads) sWcnt[i / kClasses][i % kClasses] = 0;
    __syncthreads();

    // ---- pass 1: chunk and checkpoint offsets, class histogram
    int carry_c = 0, carry_k = 0;  // the same in every thread
    for (int base = 0; base < num_seqs; base += kPrepTile) {
        const int s0 = base + t * kPrepPer;
        int nc[kPrepPer], nk[kPrepPer], sc = 0, sk = 0;
#pragma unroll
        for (int e = 0; e < kPrepPer; ++e) {
            nc[e] = 0;
            nk[e] = 0;
            if (s0 + e < num_seqs) {
                int64_t L;
                nc[e] = chunks_of(s0 + e, L);
                nk[e] = interval > 0 ? (int)(L / interval) : 0;
                atomicAdd(&sHist[length_class(nc[e])], 1);
            }
            sc += nc[e];
            sk += nk[e];
        }
        int ic = sc, ik = sk;  // inclusive scans over the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int a = __shfl_up(ic, off), b = __shfl_up(ik, off);
            if (lane >= off) {
                ic += a;
                ik += b;
            }
        }
        if (lane == 63) {
            sWsum[0][wave] = ic;
            sWsum[1][wave] = ik;
        }
        __syncthreads();
        int wc = 0, wk = 0, tc = 0, tk = 0;
#pragma unroll
        for (int w = 0; w < kPrepWaves; ++w) {
            const int a = sWsum[0][w], b = sWsum[1][w];
            wc += w < wave ? a : 0;
            wk += w < wave ? b : 0;
            tc += a;
            tk += b;
        }
        int pc = carry_c + wc + ic - sc, pk = carry_k + wk + ik - sk;
#pragma unroll
        for (int e = 0; e < kPrepPer; ++e) {
            if (s0 + e < num_seqs) {
                chunk_start[s0 + e] = pc;
                ckpt_base[s0 + e] = pk;
            }
            pc += nc[e];
            pk += nk[e];
        }
        carry_c += tc;
        carry_k += tk;
        __syncthreads();  // sWsum is rewritten by the next tile
    }
    if (t == 0) {
        chunk_start[num_seqs] = carry_c;
        ckpt_base[num_seqs] = carry_k;
    }
    if (wave == 0) {  // first slot of each class: classes in decreasing order
        const int cls = kClasses - 1 - lane;
        const int v = sHist[cls];
        int inc = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int a = __shfl_up(inc, off);
            if (lane >= off) inc += a;
        }
        sBase[cls] = inc - v;
    }
    __syncthreads();

    // ---- pass 2: order. Wave w takes sequences base + 512 w .. +511 of a
    // tile, 64 at a time in index order.
    constexpr int kPerWave = kPrepTile / kPrepWaves;
    for (int base = 0; base < num_seqs; base += kPrepTile) {
        int cls[kPrepPer], rank[kPrepPer];
#pragma unroll
        for (int i = 0; i < kPrepPer; ++i) {
            const int s = base + wave * kPerWave + 64 * i + lane;
            int c = -1;
            if (s < num_seqs) {
                int64_t L;
                c = length_class(chunks_of(s, L));
            }
            cls[i] = c;
            int r = 0;
            // one round per distinct class among the 64 lanes: rank = earlier
            // lanes of that class + the wave's count of it so far
            for (unsigned long long todo = __ballot(c >= 0); todo;) {
                const int leader = __builtin_ctzll(todo);
                const int lc = __shfl(c, leader);
                const unsigned long long same = __ballot(c == lc);
                const int before = sWcnt[wave][lc];
                if (c == lc) r = before + __popcll(same & ((1ull << lane) - 1ull));
                if (lane == leader) sWcnt[wave][lc] = before + __popcll(same);
                todo &= ~same;
            }
            rank[i] = r;
        }
        __syncthreads();
        if (t < kClasses) {  // per class: exclusive prefix over the waves, from the running slot
            int run = sBase[t];
#pragma unroll
            for (int w = 0; w < kPrepWaves; ++w) {
                const int n = sWcnt[w][t];
                sWcnt[w][t] = run;
                run += n;
            }
            sBase[t] = run;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPrepPer; ++i)
            if (cls[i] >= 0) order[sWcnt[wave][cls[i]] + rank[i]] = base + wave * kPerWave + 64 * i + lane;
        __syncthreads();
        for (int i = t; i < kPrepWaves * kClasses; i += kPrepThreads) sWcnt[i / kClasses][i % kClasses] = 0;
        __syncthreads();
    }
}

// Where a scan's chain stops to store a state: after every full checkpoint
// interval, at the start of each chunk that holds a requested position (the
// state after P tokens when P is a multiple of 64; otherwise the advance
// kernel runs the remaining P mod 64 tokens), and at the end of the sequence.
// Positions are clamped into [0, L] and list indices into [0, num_pos];
// out-of-order positions still make progress (every stop consumes an entry
// or reaches the end). All values are uniform over the workgroup.
struct StopWalk {
    const int32_t* val;
    int pj, pe, ick, next_iv, nch;
    int64_t L;
    __device__ StopWalk(const PosArgs& p, int seq, int64_t len, int64_t interval, int nchunks)
        : val(p.values), pj(0), pe(0), ick(interval > 0 ? (int)(interval / C) : 0),
          next_iv(interval > 0 ? (int)(interval / C) : 0), nch(nchunks), L(len) {
        if (p.offsets) {
            const int a = p.offsets[seq], b = p.offsets[seq + 1];
            pj = a < 0 ? 0 : (a > p.num_pos ? p.num_pos : a);
            pe = b < pj ? pj : (b > p.num_pos ? p.num_pos : b);
        }
    }
    __device__ int pos_chunk(int j) const {
        int64_t P = val[j];
        P = P < 0 ? 0 : (P > L ? L : P);
        return (int)(P / C);
    }
    __device__ int next() const {
        int s = nch;
        if (ick > 0 && next_iv < s) s = next_iv;
        if (pj < pe) {
            const int c = pos_chunk(pj);
            if (c < s) s = c;
        }
        return s;
    }
    // a checkpoint interval ends at this stop (true if it is a full one)
    __device__ bool take_interval(int stop) {
        if (ick == 0 || stop != next_iv) return false;
        next_iv += ick;
        return (int64_t)stop * C <= L;
    }
    // the next requested position whose chunk starts at this stop
    __device__ bool take_position(int stop, int& j) {
        if (pj < pe && pos_chunk(pj) == stop) {
            j = pj++;
            return true;
        }
        return false;
    }
};

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
// One workgroup per (chunk, head). Phases, separated by barriers:
//   stage   K and g into LDS (16-byte loads), beta; g floored at -kGFloor;
//           cumulative sum of g per channel in fp64, stored as G*log2(e) in
//           place of g (fp32 for bf16 inputs, fp64 for fp32 inputs); per
//           diagonal 16-row block, the channels that decay by more than
//           2^kSpanLog2 over it (slow channels, handled apart in phase A)
//   A       the 10 lower 16x16 block pairs of A (to LDS) and of P (to the
//           handoff); also the Qd, Kc^T and Gamma_last handoff
//   inverse (I + A)^-1 by forward substitution, all four waves: wave w owns
//           columns 16w..16w+15, four lanes share a column and split each
//           row's inner sum, two lane exchanges combine them
//   W       -W = -Ainv diag(beta) Kd via MFMA on W^T tiles; Ab = Ainv diag(beta)
//
// Optional parameter-free front-end (KDA's query/key L2 normalisation and
// gate activations; Kimi K3 report, "Methodology notes", Kimi Delta
// Attention): with L2 every key and query row is scaled by
// 1/sqrt(sum x^2 + 1e-6) in fp32. Key rows are rewritten normalised in LDS
// (bf16 input: as fp16 in the same 16-bit slots, so the normalised key is
// rounded once to fp16 before its MFMA operand is formed; fp32 input: fp32);
// query rows are scaled where they enter an operand. `front` bit kFrontGate
// reads g as u and uses -exp(u), bit kFrontBeta reads beta as a logit and
// uses its sigmoid.
template <int DK, bool BF16, bool L2>
__global__ __launch_bounds__(kThreads, BF16 ? 3 : (DK == 128 ? 1 : 2)) void k1_prep_kernel(
    const void* __restrict__ qin, const void* __restrict__ kin, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_start, int num_seqs, int64_t N, int H, int64_t max_chunks,
    unsigned front, unsigned char* __restrict__ handoff) {
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
    typedef TIn tin8 __attribute__((ext_vector_type(8)));

    // K is dead once phase A has built every operand that needs it, so A and
    // then Ainv reuse its LDS (K1 fits three workgroups per CU this way).
    constexpr int KBYTES = C * KP * (int)sizeof(TIn);
    constexpr int ABYTES = C * AP * (int)sizeof(float);
    __shared__ __attribute__((aligned(16))) unsigned char sKA[KBYTES > ABYTES ? KBYTES : ABYTES];
    // G * log2(e): fp32 for bf16 inputs, fp64 for fp32 inputs (whose 1e-5
    // results need differences of G exact to about 1e-9)
    using GS = typename std::conditional<BF16, float, double>::type;
    __shared__ __attribute__((aligned(16))) GS sG[C][GP];  // g, then G * log2(e)
    __shared__ __attribute__((aligned(16))) float sB[C];
    __shared__ double sTot[NQ][DK];  // cumulative-sum partial totals
    // bit c % 32 of word c / 32 of row b: channel c decays by more than
    // 2^kSpanLog2 over diagonal block b
    __shared__ unsigned sSlowCh[C / 16][NKS];
    // per wave: its diagonal block's slow channels as a list (phase A)
    static_assert(kSlowChannelsVALU % 4 == 0 && DK <= 256, "whole words of byte entries");
    __shared__ __attribute__((aligned(4))) unsigned char sSlowList[kThreads / 64][kSlowChannelsVALU];
    TIn(*sK)[KP] = reinterpret_cast<TIn(*)[KP]>(sKA);
    float(*sA)[AP] = reinterpret_cast<float(*)[AP]>(sKA);
    // inverse query-row norms (front-end) in the unused padding of G's rows:
    // a separate array took K1 over the LDS of three workgroups per CU
    static_assert(GP > DK, "G rows are padded");
    auto qn = [&](int r) -> float& { return *reinterpret_cast<float*>(&sG[r][DK]); };

    // Chunk-major, last chunk first, heads fastest: neighbouring workgroups
    // read neighbouring rows of q, k and g, and the blocks the scan needs first
    // are written last (likeliest to still be cached when it reads them).
    const int h = (int)(blockIdx.x % (unsigned)H);
    const int ci = (int)(max_chunks - 1 - (int64_t)(blockIdx.x / (unsigned)H));
    int64_t t0;
    int len;
    locate_chunk(ci, cu, chunk_start, num_seqs, N, t0, len);
    if (len <= 0) return;

    const int t = threadIdx.x;
    const int lane = t & 63;
    // wave-uniform (in a scalar register): branches and plan lookups on it
    // stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int q = lane >> 4;
    const int m = lane & 15;
    const TIn* K = static_cast<const TIn*>(kin);
    const TIn* Q = static_cast<const TIn*>(qin);
    E* hb = reinterpret_cast<E*>(handoff + ((size_t)h * max_chunks + ci) * HO::kBytes);
    float* glast = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(hb) + HO::kGlastBytes);

    auto row_off = [&](int r) -> int64_t { return ((t0 + r) * H + h) * (int64_t)DK; };
    // Input rows of this chunk: one 64-bit base, then 32-bit row offsets
    // (r * H * DK < 2^31 for r < 64); rows past the chunk end are loaded from
    // its last row (no branch) and zeroed with a select. (Measured: K1 7%
    // faster than a branch and a 64-bit offset per load; separate unclamped
    // code for full chunks was slower again.)
    const int64_t base0 = row_off(0);
    const int rstride = H * DK;
    auto row_ptr = [&](const auto* p, int r) { return p + base0 + (r < len ? r : len - 1) * rstride; };

    // ---- stage: K, g (zero past the chunk end) and beta (zero past the end).
    // Every load of the workgroup is issued before the first one is consumed.
    // Key and query rows past the chunk end hold copies of its last row and
    // need no zeroing: with beta = 0 on those rows, A, W and Ab vanish on
    // them exactly (so do U's rows, which Kc's rows multiply), no output row
    // past the end is stored, and P and A read them only at those rows.
    typedef TIn vecK_t __attribute__((ext_vector_type(VEC)));
    constexpr int KV = C * DK / VEC / kThreads;  // 16-byte K vectors per thread
    constexpr int GV = C * DK / 4 / kThreads;    // 16-byte g vectors per thread
    vecK_t kreg[KV];
    f32x4 greg[GV];
#pragma unroll
    for (int u = 0; u < KV; ++u) {
        const int i = t + u * kThreads;
        const int r = i / (DK / VEC), c = (i % (DK / VEC)) * VEC;
        const vecK_t kv = *reinterpret_cast<const vecK_t*>(row_ptr(K, r) + c);
        kreg[u] = kv;
    }
#pragma unroll
    for (int u = 0; u < GV; ++u) {
        const int i = t + u * kThreads;
        const int r = i / (DK / 4), c = (i % (DK / 4)) * 4;
        const f32x4 gv = *reinterpret_cast<const f32x4*>(row_ptr(g, r) + c);
        greg[u] = r < len ? gv : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float breg = (t < C && t < len) ? beta[(t0 + t) * H + h] : 0.f;

    // q values of the wave's phase-A row blocks, prefetched now:
    //   qa[gi][ks]: row 16*rb + m, channels 32ks + 8q .. +7
    typedef TIn tin8 __attribute__((ext_vector_type(8)));
    typedef TIn tin4 __attribute__((ext_vector_type(4)));
    // Block pairs of phase A: group gi of a wave takes row block rb with
    // column blocks sb .. sb + count - 1; group 1 is the wave's diagonal pair:
    //   wave 0: rb 3 with sb 0-1, rb 0 with sb 0    wave 1: rb 3 with sb 2,   rb 3 with sb 3
    //   wave 2: rb 2 with sb 0-1, rb 1 with sb 1    wave 3: rb 1 with sb 0,   rb 2 with sb 2
    // (every wave two row-block operand sets and at most three pairs, and
    // one diagonal block each, which may need the costlier forms below).
    // One nibble per wave in a constant, read with the uniform wave index,
    // so no table sits in memory.
    auto nib = [&](unsigned k) { return (int)((k >> (4 * wave)) & 15u); };
    auto plan_rb = [&](int gi) { return nib(gi == 0 ? 0x1233u : 0x2130u); };
    auto plan_sb = [&](int gi) { return nib(gi == 0 ? 0x0020u : 0x2130u); };
    auto plan_cnt = [&](int gi) { return nib(gi == 0 ? 0x1212u : 0x1111u); };
    tin8 qa[2][NKS];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
        const int r = 16 * plan_rb(gi) + m;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const tin8 qv = *reinterpret_cast<const tin8*>(row_ptr(Q, r) + 32 * ks + 8 * q);
            qa[gi][ks] = qv;
        }
    }
    constexpr int QDF = 4 * NKS / 4;  // Qd frags per wave
    // q values of this wave's Qd handoff frags (phase A builds them first),
    // loaded here with the rest so that their latency is hidden by the
    // cumulative sum: frag f = wave + 4i, channels 32ks + 4q .. +3 and + 16
    tin4 qd[QDF][2];
#pragma unroll
    for (int i = 0; i < QDF; ++i) {
        const int f = wave + 4 * i;
        const int rt = f / NKS, ks = f % NKS;
        const int r = 16 * rt + m;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const tin4 qv = *reinterpret_cast<const tin4*>(row_ptr(Q, r) + 32 * ks + 16 * hh + 4 * q);
            qd[i][hh] = qv;
        }
    }

#pragma unroll
    for (int u = 0; u < KV; ++u) {
        const int i = t + u * kThreads;
        const int r = i / (DK / VEC), c = (i % (DK / VEC)) * VEC;
        *reinterpret_cast<vecK_t*>(&sK[r][c]) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < GV; ++u) {
        const int i = t + u * kThreads;
        const int r = i / (DK / 4), c = (i % (DK / 4)) * 4;
        f32x4 gv = greg[u];
        if ((front & kFrontGate) && r < len) {  // g = -exp(u); rows past the end stay 0
#pragma unroll
            for (int e = 0; e < 4; ++e) gv[e] = -__expf(gv[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) gv[e] = fmaxf(gv[e], BF16 ? -kGFloorBF16 : -kGFloorF32);
        if constexpr (BF16) {
            *reinterpret_cast<f32x4*>(&sG[r][c]) = gv;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) sG[r][c + e] = (double)gv[e];
        }
    }
    if (t < C) sB[t] = ((front & kFrontBeta) && t < len) ? 1.f / (1.f + __expf(-breg)) : breg;
    // inverse query-row norms from this wave's phase-A rows: the four lanes
    // m + 16q hold the channels of row 16 rb + m between them
    if constexpr (L2) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            const int rb = plan_rb(gi);
            float ss = 0.f;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = qf_in<TIn>(qa[gi][ks][e]);
                    ss += x * x;
                }
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            if (q == 0) qn(16 * rb + m) = 1.f / sqrtf(ss + kL2Eps);  // rows shared by two waves get equal values
        }
    }
    __syncthreads();
    {
        // inclusive cumulative sum per channel (rows past the end add 0)
        const int c = t % DK, grp = t / DK;
        double acc = 0;
#pragma unroll
        for (int r = grp * RPQ; r < (grp + 1) * RPQ; ++r) acc += (double)sG[r][c];
        sTot[grp][c] = acc;
        if constexpr (L2) {  // key rows normalised in place: four threads per row
            constexpr int NV = DK / 4 / VEC;  // 16-byte vectors per thread
            const int r = t >> 2, part = t & 3;
            vecK_t* row = reinterpret_cast<vecK_t*>(&sK[r][part * (DK / 4)]);
            vecK_t kv[NV];
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                kv[j] = row[j];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float x = qf_in<TIn>(kv[j][e]);
                    ss += x * x;
                }
            }
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            const float inv = 1.f / sqrtf(ss + kL2Eps);
#pragma unroll
            for (int j = 0; j < NV; ++j) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float x = qf_in<TIn>(kv[j][e]) * inv;
                    if constexpr (BF16) kv[j][e] = __builtin_bit_cast(unsigned short, (_Float16)x);
                    else kv[j][e] = x;
                }
                row[j] = kv[j];
            }
        }
        __syncthreads();
        double run = 0;
        for (int p = 0; p < grp; ++p) run += sTot[p][c];
        static_assert(RPQ % 16 == 0, "a row group holds whole 16-row blocks");
    static_assert(DK % 64 == 0, "a wave's channels lie in one row group");
        GS first = 0;
#pragma unroll
        for (int i = 0; i < RPQ; ++i) {
            const int r = grp * RPQ + i;
            run += (double)sG[r][c];
            const GS val = (GS)(run * 1.4426950408889634);
            sG[r][c] = val;
            // decay over the 16-row block in this channel (G is non-increasing)
            if (i % 16 == 0) first = val;
            if (i % 16 == 15) {
                // a wave holds 64 consecutive channels of one row group: its
                // vote is two whole words of the block's channel mask
                const unsigned long long vote =
                    __ballot(first - val > (GS)(BF16 ? kSpanLog2BF16 : kSpanLog2F32));
                if (lane == 0) {
                    const int b = grp * (RPQ / 16) + i / 16;
                    sSlowCh[b][c / 32] = (unsigned)vote;
                    sSlowCh[b][c / 32 + 1] = (unsigned)(vote >> 32);
                }
            }
        }
    }
    __syncthreads();

    auto kval = [&](int r, int c) -> float {  // key value (normalised fp16 bits: L2 and bf16)
        if constexpr (L2 && BF16) return (float)__builtin_bit_cast(_Float16, sK[r][c]);
        else return qf_in<TIn>(sK[r][c]);
    };
    auto qf = [&](TIn v) -> float {
        if constexpr (BF16) return bf16_to_f32(v);
        else return v;
    };
    // (G_a - G_b) * log2(e) in channel c, differenced in the stored precision
    auto gdiff = [&](int a, int b, int c) -> float { return (float)(sG[a][c] - sG[b][c]); };

    f32x4 aT[3];  // A tiles of this wave's block pairs: group 0 in slots 0-1, the diagonal in 2

    // ---- phase A: 16x16 block pairs (rb, sb), sb <= rb, reference row 16*rb:
    // every factor e^(G_r - G_ref) (r >= ref) is <= 1 and e^(G_ref - G_s) is
    // <= 1 for s < ref. Waves take the pairs grouped by rb so the row-block
    // operands X = Kd', Z = Qd' are built once per rb. The wave's diagonal
    // block (group 1) may hold slow channels: up to kSlowChannelsVALU of them
    // are left out of its products and their pairs summed on the vector
    // units; with more the pair takes the four-level products instead.
    const int drb = plan_rb(1);
    unsigned dmask[NKS];  // the diagonal block's slow channels (wave-uniform)
    int nslow = 0;
#pragma unroll
    for (int w = 0; w < NKS; ++w) {
        dmask[w] = __builtin_amdgcn_readfirstlane(sSlowCh[drb][w]);
        nslow += __builtin_popcount(dmask[w]);
    }
    const bool dfour = nslow > kSlowChannelsVALU;
    {
        // A[r'][s'] with r' = 16rb + 4q + i, s' = 16sb + m, kept in registers
        // until every wave is done reading K; P^T[s'][r'] with s' = 16sb + 4q + i,
        // r' = 16rb + m -> P A-frag [rt = rb][slab sb/2], slots 4*(sb%2) + i of
        // lane (m + 16q). Stores P and returns the A tile (times beta, strictly
        // lower part).
        auto store_pair = [&](int rb, int sb, const f32x4& accA, const f32x4& accP) -> f32x4 {
            // beta of rows 16 rb + 4q .. +3, read whole (a conditional read per
            // element became a branch and an LDS round trip each)
            const f32x4 bv = *reinterpret_cast<const f32x4*>(&sB[16 * rb + 4 * q]);
            f32x4 at;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * rb + 4 * q + i, ss = 16 * sb + m;
                at[i] = ss < rr ? bv[i] * accA[i] : 0.f;
            }
            typedef E e4 __attribute__((ext_vector_type(4)));
            e4 pv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ss = 16 * sb + 4 * q + i, rr = 16 * rb + m;
                pv[i] = (E)(ss <= rr ? accP[i] : 0.f);
            }
            *reinterpret_cast<e4*>(hb + HO::kP + ((size_t)HO::tri(rb, sb / 2) * 64 + lane) * 8 + 4 * (sb % 2)) = pv;
            return at;
        };
        // Qd A-frags (first, so that the prefetched queries die early): rows tokens (tile rt), K channels (slab ks, permuted)
#pragma unroll
        for (int i = 0; i < QDF; ++i) {
            const int f = wave + 4 * i;
            const int rt = f / NKS, ks = f % NKS;
            const int r = 16 * rt + m;
            // perm32(q, e): channels 32ks + 4q + e (e < 4) and 32ks + 16 + 4q + e - 4
            Frag out;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 32 * ks + perm32(q, e);
                out[e] = (E)(qf(qd[i][e >> 2][e & 3]) * (L2 ? qn(r) : 1.f) * fast_exp2((float)sG[r][c]));
            }
            store_frag<Frag, E>(hb + HO::kQd, rt * NKS + ks, lane, out);
        }
        // Group 0: off-diagonal pairs.
        {
            const int rb = plan_rb(0);
            const int ref = 16 * rb;
            const int r = 16 * rb + m;
            const float zq = L2 ? qn(r) : 1.f;
            Frag X[NKS], Z[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int c = 32 * ks + 8 * q + e;
                    const float fr = fast_exp2(gdiff(r, ref, c));
                    X[ks][e] = (E)(kval(r, c) * fr);
                    Z[ks][e] = (E)(qf(qa[0][ks][e]) * zq * fr);
                }
            }
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                if (k2 >= plan_cnt(0)) break;
                const int sb = plan_sb(0) + k2;
                const int s = 16 * sb + m;
                f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    Frag Y;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int c = 32 * ks + 8 * q + e;
                        Y[e] = (E)(kval(s, c) * fast_exp2(gdiff(ref, s, c)));
                    }
                    accA = M::run(X[ks], Y, accA);  // rows r, cols s
                    accP = M::run(Y, Z[ks], accP);  // P^T: rows s, cols r
                }
                aT[k2] = store_pair(rb, sb, accA, accP);
            }
        }
        // Group 1: the diagonal pair (r and s both run over rows 16 drb + m).
        {
            const int ref = 16 * drb;
            const int r = ref + m;
            const float zq = L2 ? qn(r) : 1.f;
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            // reference row 16 drb; slow channels are zero in the operand both
            // products share (their factors may not fit it), a select only
            // compiled into the copy for blocks that have them
            auto diag_products = [&](auto masked) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const unsigned lb = dmask[ks] >> (8 * q);  // this lane's 8 channels
                    Frag X, Y, Z;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int c = 32 * ks + 8 * q + e;
                        const float d = gdiff(r, ref, c);
                        const float kv = kval(r, c);
                        const float fr = fast_exp2(d);
                        X[e] = (E)(kv * fr);
                        Z[e] = (E)(qf(qa[1][ks][e]) * zq * fr);
                        const E y = (E)(kv * fast_exp2(-d));
                        if constexpr (decltype(masked)::value) Y[e] = ((lb >> e) & 1u) ? (E)0.f : y;
                        else Y[e] = y;
                    }
                    accA = M::run(X, Y, accA);  // rows r, cols s
                    accP = M::run(Y, Z, accP);  // P^T: rows s, cols r
                }
            };
            if (nslow == 0) diag_products(std::false_type{});
            else if (!dfour) diag_products(std::true_type{});
            if (nslow && !dfour) {
                // The slow channels' pairs exactly, in fp32 on the vector
                // units: A tile element i is the pair (r = 4q + i, s = m) when
                // 4q + i > m, P^T tile element i the pair (s = 4q + i, r = m)
                // otherwise; either way its factor is 2^-|G_4q+i - G_m| (G is
                // non-increasing) times k_4q+i, and the other term k_m or q_m.
                // The query of row m is held by lane m + 16 ((c % 32) / 8)
                // (prefetched, element (c / 32, c % 8)): a uniformly indexed
                // register read and a lane exchange. Four channels at a time;
                // those past the last one get zero terms.
                constexpr int QW = (int)sizeof(tin8) / 4;  // dwords per tin8
                typedef unsigned qwords_t __attribute__((ext_vector_type(NKS * QW)));
                typedef unsigned tin8w_t __attribute__((ext_vector_type(QW)));
                qwords_t qw;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const tin8w_t v = __builtin_bit_cast(tin8w_t, qa[1][ks]);
#pragma unroll
                    for (int j = 0; j < QW; ++j) qw[ks * QW + j] = v[j];
                }
                // the channel list: lane l places channel 64h + l at its rank
                // among the block's slow channels
                {
                    int base = 0;
#pragma unroll
                    for (int hw = 0; hw < NKS / 2; ++hw) {
                        const unsigned lo = dmask[2 * hw], hi = dmask[2 * hw + 1];
                        const int rank = base + (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
                        const unsigned long long word = ((unsigned long long)hi << 32) | lo;
                        if ((word >> lane) & 1ull) sSlowList[wave][rank] = (unsigned char)(64 * hw + lane);
                        base += __builtin_popcountll(word);
                    }
                    // written and read by this wave only
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                }
                bool up[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) up[i] = 4 * q + i > m;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
                for (int j0 = 0; j0 < nslow; j0 += 4) {
                    // four entries (bytes past the list's end are stale: masked
                    // into range, their terms zero)
                    const unsigned w4 = __builtin_amdgcn_readfirstlane(
                        *reinterpret_cast<const unsigned*>(&sSlowList[wave][j0]));
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool ok = j0 + j < nslow;
                        const int c = (int)((w4 >> (8 * j)) & (unsigned)(DK - 1));
                        const int el = (c >> 5) * 8 + (c & 7);  // element of qa[1][.][.]
                        const unsigned dw = qw[BF16 ? el >> 1 : el];
                        const unsigned got = (unsigned)__shfl((int)dw, m + 16 * ((c & 31) >> 3));
                        float qv;
                        if constexpr (BF16) qv = bf16_to_f32((unsigned short)((c & 1) ? got >> 16 : got & 0xffffu));
                        else qv = __uint_as_float(got);
                        const float okf = ok ? 1.f : 0.f;  // a factor, not a branch around the loads
                        const float km = kval(r, c) * okf;
                        const float qm = qv * (zq * okf);
                        const GS gm = sG[r][c];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int rr = ref + 4 * q + i;
                            const float d = (float)(sG[rr][c] - gm);
                            const float tk = kval(rr, c) * fast_exp2(-fabsf(d));
                            acc[i] = fmaf(tk, up[i] ? km : qm, acc[i]);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    accA[i] += up[i] ? acc[i] : 0.f;
                    accP[i] += up[i] ? 0.f : acc[i];
                }
            } else if (dfour) {
                // Four levels h = 8, 4, 2, 1 over the local row index
                // (lane row m): rows with bit h set (r side) take
                // e^(G_m - G_{m & ~(h-1)}), rows with bit h clear (s side)
                // take e^(G_{(m & ~(h-1)) + h} - G_m); both are <= 1, and
                // for r, s in one 2h-run on opposite sides of its middle
                // their product is e^(G_r - G_s). Each level keeps only
                // those pairs; P's diagonal (factor 1) is added at the end.
#pragma unroll 1
                for (int lv = 0; lv < 4; ++lv) {
                    const int hh = 8 >> lv;
                    const bool up = (m & hh) != 0;
                    const int oth = ref + (m & ~(hh - 1)) + (up ? 0 : hh);
                    // factor 2^(G_ga - G_gb) <= 1: the rows are chosen per
                    // lane once, so each element needs no select of its sign
                    const int ga = up ? r : oth, gb = up ? oth : r;
                    f32x4 tA = {0.f, 0.f, 0.f, 0.f}, tP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        Frag kf, qf8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int c = 32 * ks + 8 * q + e;
                            const float f = fast_exp2(gdiff(ga, gb, c));
                            kf[e] = (E)(kval(r, c) * f);
                            qf8[e] = (E)(qf(qa[1][ks][e]) * zq * f);
                        }
                        // Every lane's row enters both sides unmasked: the
                        // products of two r-side or two s-side rows (all
                        // factors <= 1, so finite) are dropped below with
                        // the pairs outside the level
                        tA = M::run(kf, kf, tA);   // rows r, cols s
                        tP = M::run(kf, qf8, tP);  // P^T: rows s, cols r
                        __builtin_amdgcn_sched_barrier(0);  // one slab's operands live at a time
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ra = 4 * q + i;  // A tile: row ra, column m
                        accA[i] += (((ra ^ m) < 2 * hh) && (ra & hh) && !(m & hh)) ? tA[i] : 0.f;
                        const int sp = 4 * q + i;  // P^T tile: row sp (s), column m (r)
                        accP[i] += (((sp ^ m) < 2 * hh) && (m & hh) && !(sp & hh)) ? tP[i] : 0.f;
                    }
                }
                float dq = 0.f;  // q_r . k_r over this lane's channels, then all four lanes of row m
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) dq += qf(qa[1][ks][e]) * kval(r, 32 * ks + 8 * q + e);
                dq = pair_sum32(pair_sum16(dq)) * zq;
#pragma unroll
                for (int i = 0; i < 4; ++i) accP[i] += (4 * q + i == m) ? dq : 0.f;
            }
            aT[2] = store_pair(drb, drb, accA, accP);
        }
        // zero halves inside stored slabs: (rb, sb) = (0, 1) and (2, 3)
        if (wave == 2 || wave == 3) {
            const int rb = wave == 2 ? 0 : 2, sb = rb + 1;
            typedef E e4 __attribute__((ext_vector_type(4)));
            *reinterpret_cast<e4*>(hb + HO::kP + ((size_t)HO::tri(rb, sb / 2) * 64 + lane) * 8 + 4 * (sb % 2)) = e4{};
        }
        // The slabs (row tiles 0-1, token slab 1) of P and Ab lie wholly
        // above the diagonal: they are zero, and neither stored nor read.
        // Kc^T A-frags: rows channels (tile ct), K tokens (slab ts, permuted)
        for (int f = wave; f < NRT * 2; f += 4) {
            const int ct = f / 2, ts = f % 2;
            const int c = 16 * ct + m;
            Frag out;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = 32 * ts + perm32(q, e);
                out[e] = (E)(kval(r, c) * fast_exp2(gdiff(C - 1, r, c)));
            }
            store_frag<Frag, E>(hb + HO::kKc, ct * 2 + ts, lane, out);
        }
        for (int c = t; c < DK; c += kThreads) glast[c] = fast_exp2((float)sG[C - 1][c]);
    }
    // (beta Kd)^T operands of phase C, built while K is still in LDS:
    // row c = 16(2ks + half) + m, K index s = 32ts + 8q + e, ks = wave % NKS
    Frag aF[2][2];
    {
        const int ks = wave % NKS;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int ts = 0; ts < 2; ++ts) {
                const int c = 16 * (2 * ks + half) + m;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = 32 * ts + 8 * q + e;
                    aF[half][ts][e] = (E)(sB[s] * kval(s, c) * fast_exp2((float)sG[s][c]));
                }
            }
    }
    __syncthreads();

    // K is no longer read: the A tiles go to its LDS
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
        if (k2 >= plan_cnt(0)) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) sA[16 * plan_rb(0) + 4 * q + i][16 * (plan_sb(0) + k2) + m] = aT[k2][i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sA[16 * drb + 4 * q + i][16 * drb + m] = aT[2][i];
    __syncthreads();

    // ---- inverse: X = (I + A)^-1 in 16x16 blocks (all fp32).
    // (1) wave b inverts the unit lower-triangular diagonal block I + A_bb by
    //     forward substitution: lane (c = m, p = q) owns column c and sums the
    //     terms s = 4u + p of each row; the four partial sums are combined with
    //     two lane-pair exchanges (identical order in every lane). In place.
    {
        const int b = wave, c = m, p = q;
        float xs[4] = {0.f, 0.f, 0.f, 0.f};  // xs[u] = x[4u + p][c]
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (4 * u < r) acc += sA[16 * b + r][16 * b + 4 * u + p] * xs[u];  // A_bb[r][s >= r] = 0
            acc = pair_sum16(acc);
            acc = pair_sum32(acc);
            const float xr = (r == c ? 1.f : 0.f) - acc;
            // lane p keeps rows 4u + p: xs[r >> 2] is still 0 in every lane
            // that does not keep row r, so a masked add stores it without a
            // branch (a branch here split the substitution into one block per
            // row, and no LDS read could be issued ahead of its row)
            xs[r >> 2] += (p == (r & 3) ? 1.f : 0.f) * xr;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) sA[16 * b + 4 * u + p][16 * b + c] = xs[u];
    }
    __syncthreads();
    // (2) off-diagonal blocks, X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj, by
    //     distance i - j = 1, 2, 3 on v_mfma_f32_16x16x4_f32. K index of
    //     instruction e in lane group g is 4g + e, so a result tile is the next
    //     product's B operand as it stands. X_ij (i > j) is parked transposed
    //     in the free upper block (j, i) until A is no longer needed.
    {
        auto mma_acc = [&](f32x4 acc, int i, int k, int j) -> f32x4 {  // acc += A_ik X_kj
            const f32x4 av = *reinterpret_cast<const f32x4*>(&sA[16 * i + m][16 * k + 4 * q]);
            f32x4 bv;
            if (k == j) {
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[e] = sA[16 * j + 4 * q + e][16 * j + m];
            } else {
                bv = *reinterpret_cast<const f32x4*>(&sA[16 * j + m][16 * k + 4 * q]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc, 0, 0, 0);
            return acc;
        };
        auto finish = [&](const f32x4& T, int i, int j) {  // X_ij = -X_ii T, stored transposed
            const f32x4 av = *reinterpret_cast<const f32x4*>(&sA[16 * i + m][16 * i + 4 * q]);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], T[e], acc, 0, 0, 0);
            *reinterpret_cast<f32x4*>(&sA[16 * j + m][16 * i + 4 * q]) = -acc;
        };
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        if (wave < 3) {  // (1,0), (2,1), (3,2)
            const int i = wave + 1, j = wave;
            finish(mma_acc(z, i, j, j), i, j);
        }
        __syncthreads();
        if (wave < 2) {  // (2,0), (3,1)
            const int i = wave + 2, j = wave;
            finish(mma_acc(mma_acc(z, i, j, j), i, j + 1, j), i, j);
        }
        __syncthreads();
        if (wave == 0)  // (3,0)
            finish(mma_acc(mma_acc(mma_acc(z, 3, 0, 0), 3, 1, 0), 3, 2, 0), 3, 0);
        __syncthreads();
        // move the parked blocks into the lower triangle and clear the upper
        // one: thread t takes element (r, c) of every block. All six reads
        // are issued before any write (one LDS round trip instead of six);
        // no thread reads an element another thread writes.
        static_assert(kThreads == 256, "one element per thread and block");
        constexpr int blocks[6][2] = {{1, 0}, {2, 1}, {3, 2}, {2, 0}, {3, 1}, {3, 0}};
        const int r = t >> 4, c = t & 15;
        float val[6];
#pragma unroll
        for (int b = 0; b < 6; ++b) val[b] = sA[16 * blocks[b][1] + c][16 * blocks[b][0] + r];
#pragma unroll
        for (int b = 0; b < 6; ++b) {
            const int i = blocks[b][0], j = blocks[b][1];
            sA[16 * j + c][16 * i + r] = 0.f;
            sA[16 * i + r][16 * j + c] = val[b];
        }
    }
    __syncthreads();

    // ---- phase C: -W from W^T = (diag(beta) Kd)^T Ainv^T and the Ab handoff.
    // W^T tiles (channel tile ct, token tile rt); tiles 2ks and 2ks+1 of the
    // same rt stack into the W A-frag of (rt, slab ks). Each wave keeps one ks.
    {
        const int ks = wave % NKS;
        for (int f = wave; f < 4 * NKS; f += 4) {
            const int rt = f / NKS;
            f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            const int nts = rt >= 2 ? 2 : 1;  // Ainv[r][s] = 0 for s > r
            for (int ts = 0; ts < nts; ++ts) {
                Frag b;  // Ainv^T: column r = 16rt + m, K = s = 32ts + 8q + e
                const int r = 16 * rt + m;
                const f32x4 b0 = *reinterpret_cast<const f32x4*>(&sA[r][32 * ts + 8 * q]);
                const f32x4 b1 = *reinterpret_cast<const f32x4*>(&sA[r][32 * ts + 8 * q + 4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    b[e] = (E)b0[e];
                    b[4 + e] = (E)b1[e];
                }
                acc[0] = M::run(aF[0][ts], b, acc[0]);
                acc[1] = M::run(aF[1][ts], b, acc[1]);
            }
            Frag out;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                out[i] = (E)(-acc[0][i]);
                out[4 + i] = (E)(-acc[1][i]);
            }
            store_frag<Frag, E>(hb + HO::kW, rt * NKS + ks, lane, out);
        }
    }
    // Ab = Ainv diag(beta) A-frags: rows tokens (tile rt), K tokens (slab ts, permuted);
    // slabs (rt 0-1, ts 1) are identically zero and not stored.
    {
        // frags (rt, ts): (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
        for (int f = wave; f < 6; f += 4) {
            const int rt = f < 2 ? f : (f >> 1) + 1, ts = f < 2 ? 0 : (f & 1);
            const int r = 16 * rt + m;
            Frag out;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = 32 * ts + perm32(q, e);
                out[e] = (E)(sA[r][s] * sB[s]);
            }
            store_frag<Frag, E>(hb + HO::kAb, f, lane, out);  // f = HO::tri(rt, ts)
        }
    }
}

// ---------------------------------------------------------------- K2 -----
// Per-wave operands of one chunk: -W, Qd (row tile = wave), Ab, P (row tile =
// wave; both token slabs, the second is zero for row tiles 0-1), Kc^T (the
// wave's state row tiles), Gamma_last for those rows, and this thread's share
// of the V tile.
template <int DK, int NT, bool BF16>
struct ChunkOps {
    using Frag = typename Mma<BF16>::Frag;
    using TIn = typename std::conditional<BF16, unsigned short, float>::type;
    typedef TIn tin4 __attribute__((ext_vector_type(4)));
    static constexpr int NKS = DK / 32;
    static constexpr int TPW = DK / 64;
    Frag ab[2], wn[NKS], qd[NKS], p[2], kc[TPW][2];
    f32x4 gl[TPW];
    tin4 v[NT];
};

// One workgroup = one (sequence, head) and 16*NT value columns; wave w owns
// U/O row tile w (tokens 16w..16w+15) and state row tiles w*TPW .. +TPW-1.
// The operands of chunk n + 2 are requested while chunk n computes, in three
// rotating register buffers. The chunk loop has no branches (loads are
// unconditional, a token past the end of a sequence stores to a sink), so the
// compiler's memory-wait analysis stays exact and the prefetches stay in
// flight; outputs leave as one 16-byte store per lane and 16-column tile.
template <int DK, int DV, int NT, bool BF16>
__global__ __launch_bounds__(kThreads) void k2_scan_kernel(
    const void* __restrict__ vin, const int32_t* __restrict__ cu, const int32_t* __restrict__ order,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ ckpt_base, int npairs,
    int64_t N, int H, int64_t max_chunks, const unsigned char* __restrict__ handoff,
    const float* __restrict__ s0, float* __restrict__ sfinal, int64_t interval,
    float* __restrict__ ckpt, int64_t ckpt_rows, PosArgs pos, float* __restrict__ o,
    float* __restrict__ sink) {
    using M = Mma<BF16>;
    using E = typename M::E;
    using Frag = typename M::Frag;
    using TIn = typename std::conditional<BF16, unsigned short, float>::type;
    using HO = Handoff<DK, BF16>;
    using Ops = ChunkOps<DK, NT, BF16>;
    using tin4 = typename Ops::tin4;
    typedef E e4 __attribute__((ext_vector_type(4)));
    constexpr int NKS = DK / 32;
    constexpr int TPW = DK / 64;            // state row tiles per wave
    constexpr int NVB = DV / (16 * NT);     // value-column blocks per (seq, head)
    constexpr int NV = 16 * NT;

    __shared__ __attribute__((aligned(32))) E sS[NKS][NT][64][8];  // S(n) as B-frags
    __shared__ __attribute__((aligned(32))) E sV[2][NT][64][8];    // V(n) as B-frags
    __shared__ __attribute__((aligned(32))) E sU[2][NT][64][8];    // U(n) as B-frags

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
    const int64_t cpbase = ckpt_base ? ckpt_base[seq] : 0;  // one sequence: base 0

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int q = lane >> 4;
    const int m = lane & 15;
    const int rt = wave;                  // U / O row tile
    const TIn* V = static_cast<const TIn*>(vin);
    // V tile: thread t stages token vs = t / 4, columns 16ct + 4*(t % 4) .. +3
    const int vs = t >> 2, vc = 4 * (t & 3);
    // this lane's private sink slot (stores that must not land anywhere)
    float* my_sink = sink + ((size_t)(id & (kSinkSlots - 1)) * kThreads + t) * kSinkFloats;
    const unsigned char* hbase = handoff + ((size_t)h * max_chunks + cbase) * HO::kBytes;

    // Issue the loads of chunk n (0 <= n < nch: in bounds) in four groups, so a
    // step can spread them over its phases instead of filling the memory
    // queue in one burst (a wave issues in order: a full queue would stall
    // its arithmetic behind its own prefetches).
    auto load_ops = [&](Ops& op, int n, int grp) {
        const E* hb = reinterpret_cast<const E*>(hbase + (size_t)n * HO::kBytes);
        if (grp == 0) {
            op.ab[0] = load_frag<Frag, E>(hb + HO::kAb, HO::tri(rt, 0), lane);
            op.p[0] = load_frag<Frag, E>(hb + HO::kP, HO::tri(rt, 0), lane);
            if (rt >= 2) {  // token slab 1 of row tiles 0-1 is zero (not stored)
                op.ab[1] = load_frag<Frag, E>(hb + HO::kAb, HO::tri(rt, 1), lane);
                op.p[1] = load_frag<Frag, E>(hb + HO::kP, HO::tri(rt, 1), lane);
            } else {
                op.ab[1] = Frag{};
                op.p[1] = Frag{};
            }
        } else if (grp == 1) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) op.wn[ks] = load_frag<Frag, E>(hb + HO::kW, rt * NKS + ks, lane);
        } else if (grp == 2) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) op.qd[ks] = load_frag<Frag, E>(hb + HO::kQd, rt * NKS + ks, lane);
        } else {
            const float* glast = reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(hb) + HO::kGlastBytes);
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int srt = wave * TPW + i;
                op.kc[i][0] = load_frag<Frag, E>(hb + HO::kKc, srt * 2 + 0, lane);
                op.kc[i][1] = load_frag<Frag, E>(hb + HO::kKc, srt * 2 + 1, lane);
                op.gl[i] = *reinterpret_cast<const f32x4*>(glast + 16 * srt + 4 * q);
            }
            // token rows past the end read the last valid row (zeroed when staged)
            const int64_t left = L - (int64_t)n * C;
            const int64_t tok = tstart + (int64_t)n * C + (vs < left ? vs : left - 1);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
                op.v[ct] = *reinterpret_cast<const tin4*>(V + (tok * H + h) * (int64_t)DV + j0 + 16 * ct + vc);
        }
    };
    auto load_all = [&](Ops& op, int n) {
        load_ops(op, n, 0);
        load_ops(op, n, 1);
        load_ops(op, n, 2);
        load_ops(op, n, 3);
    };

    // state rows owned: channel 16*srt + 4q + i, column j0 + 16ct + m
    f32x4 S[TPW][NT];
    const size_t sbase = ((size_t)seq * H + h) * DK * DV;
    if (s0) {
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    S[i][ct][ii] = s0[sbase + (size_t)(16 * (wave * TPW + i) + 4 * q + ii) * DV + j0 + 16 * ct + m];
    } else {
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) S[i][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    auto store_state = [&](float* dst) {
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    dst[(size_t)(16 * (wave * TPW + i) + 4 * q + ii) * DV + j0 + 16 * ct + m] = S[i][ct][ii];
    };

    // One chunk step with operands `cur` (chunk n), prefetching chunk `pn` into `nxt`.
    auto step = [&](const Ops& cur, int n, Ops& nxt, int pn) {
        load_ops(nxt, pn, 0);
        const int64_t tok0 = tstart + (int64_t)n * C;
        const int64_t left = L - (int64_t)n * C;
        const int len = left < C ? (int)left : C;

        // (a) publish S as B-frags (slab = row tile / 2, half = row tile % 2) and the V tile
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int srt = wave * TPW + i;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                e4 v4;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) v4[ii] = (E)S[i][ct][ii];
                *reinterpret_cast<e4*>(&sS[srt / 2][ct][lane][4 * (srt % 2)]) = v4;
            }
        }
        {
            // token vs -> slab vs/32, B-frag lane (col & 15) + 16 * qq, slot ee (inverse of perm32)
            const int ts = vs >> 5, w32 = vs & 31;
            const int qq = (w32 & 15) >> 2;
            const int ee = (w32 & 3) + ((w32 >> 4) << 2);
            const bool valid = vs < len;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    float val;
                    if constexpr (BF16) val = bf16_to_f32(cur.v[ct][cc]);
                    else val = cur.v[ct][cc];
                    sV[ts][ct][vc + cc + 16 * qq][ee] = (E)(valid ? val : 0.f);
                }
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        load_ops(nxt, pn, 1);
        __builtin_amdgcn_sched_barrier(0);

        // (c) U = Ab V - W S ; O^T = S^T Qd^T  (row tile = wave). A B-operand
        // fragment of X (K x N) is also the A-operand fragment of X^T, so O^T
        // takes the same fragments with the operands swapped; its result tile
        // gives each lane 4 adjacent value columns of one token (16-byte stores).
        // The LDS fragments (V by slab, then S by K slab, column tile fastest)
        // are read PD ahead of their products, so no product waits for a
        // fresh LDS round trip.
        f32x4 U[NT], O[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            U[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            O[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        {
            // fragment k: V slab k / NT for k < 2 NT, else S slab k / NT - 2; column tile k % NT
            constexpr int NR = (2 + NKS) * NT, PD = NT * 2 < NR ? NT * 2 : NR;
            auto rd = [&](int k) -> Frag {
                const int sl = k / NT, ct = k % NT;
                return sl < 2 ? *reinterpret_cast<const Frag*>(&sV[sl][ct][lane][0])
                              : *reinterpret_cast<const Frag*>(&sS[sl - 2][ct][lane][0]);
            };
            Frag pf[PD];
            static_for<PD>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                pf[k] = rd(k);
            });
            static_for<NR>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                const Frag f = pf[k % PD];
                if constexpr (k + PD < NR) pf[k % PD] = rd(k + PD);
                constexpr int sl = k / NT, ct = k % NT;
                if constexpr (sl < 2) {
                    U[ct] = M::run(cur.ab[sl], f, U[ct]);
                } else {
                    U[ct] = M::run(cur.wn[sl - 2], f, U[ct]);
                    O[ct] = M::run(f, cur.qd[sl - 2], O[ct]);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        // (d) publish U as B-frags (K = tokens): slab rt/2, half rt%2
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            e4 u4;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) u4[ii] = (E)U[ct][ii];
            *reinterpret_cast<e4*>(&sU[rt / 2][ct][lane][4 * (rt % 2)]) = u4;
        }
        __builtin_amdgcn_sched_barrier(0);
        load_ops(nxt, pn, 2);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        load_ops(nxt, pn, 3);
        __builtin_amdgcn_sched_barrier(0);

        // (g) S <- diag(Gamma_last) S + Kc^T U  (on the dependency chain: first),
        // every U fragment read before the first product
        Frag uf[2][NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            uf[0][ct] = *reinterpret_cast<const Frag*>(&sU[0][ct][lane][0]);
            uf[1][ct] = *reinterpret_cast<const Frag*>(&sU[1][ct][lane][0]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                f32x4 a = S[i][ct] * cur.gl[i];
                a = M::run(cur.kc[i][0], uf[0][ct], a);
                a = M::run(cur.kc[i][1], uf[1][ct], a);
                S[i][ct] = a;
            }

        // (f) O^T += U^T P^T; lane (m, q) holds token 16*rt + m, columns 4q .. 4q+3
        // of each 16-column tile: one 16-byte store per tile (a token past the
        // end of the sequence stores to the sink)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            O[ct] = M::run(uf[0][ct], cur.p[0], O[ct]);
            O[ct] = M::run(uf[1][ct], cur.p[1], O[ct]);
        }
        {
            const int tok = 16 * rt + m;
            float* op = tok < len ? o + ((tok0 + tok) * H + h) * (int64_t)DV + j0 + 4 * q : my_sink;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
                *reinterpret_cast<f32x4*>(op + (tok < len ? 16 * ct : 0)) = O[ct];
        }

    };

    // Chunks run in segments that end on checkpoint boundaries, so the
    // branch-free chunk loop never stores a state; each checkpoint is written
    // between segments. Without checkpoints there is one segment.
    StopWalk sw(pos, seq, L, interval, nch);
    int64_t cidx = cpbase;
    Ops b0, b1, b2;
    for (int n0 = 0;;) {
        const int stop = sw.next();
        if (stop > n0) {
            const int seg0 = n0, seg1 = stop;
            load_all(b0, seg0);
            load_all(b1, seg0 + 1 < seg1 ? seg0 + 1 : seg0);
            for (int n = seg0; n < seg1; n += 3) {
                step(b0, n, b2, n + 2 < seg1 ? n + 2 : seg1 - 1);
                if (n + 1 >= seg1) break;
                step(b1, n + 1, b0, n + 3 < seg1 ? n + 3 : seg1 - 1);
                if (n + 2 >= seg1) break;
                step(b2, n + 2, b1, n + 4 < seg1 ? n + 4 : seg1 - 1);
            }
            n0 = stop;
        }
        if (sw.take_interval(stop)) {  // a full interval ends here: checkpoint
            if (cidx < ckpt_rows) store_state(ckpt + (cidx * H + h) * (size_t)DK * DV);
            ++cidx;
        }
        for (int j; sw.take_position(stop, j);)
            store_state(pos.states + ((size_t)j * H + h) * DK * DV);
        if (stop >= nch) break;
    }

    if (sfinal) store_state(sfinal + sbase);
}

// Three-wave scan: one workgroup = one (sequence, head) and 16 value columns,
// with the whole state slice (DK x 16) in the registers of wave 0.
//   wave 0  the chain: U = U0 - W S, then S <- diag(Gamma_last) S + Kc^T U.
//           S and U pass from one product to the next inside the lane that
//           holds them (the K-slab permutation): no LDS round trip.
//   wave 1  runs two chunks ahead: stages a chunk's V tile, forms U0 = Ab V
//           and Gamma_last for wave 0 (which reads them one step ahead, so no
//           LDS latency sits on the chain), and touches the lines of the chunk
//           five steps ahead so that the operand loads of all waves hit L2.
//   wave 2  trails by one chunk: O^T = S^T Qd^T + U^T P^T from the S and U
//           fragments wave 0 leaves in LDS, one 16-byte store per lane.
// One barrier per chunk; the S/U fragments are double-buffered by chunk
// parity, U0 and Gamma_last triple-buffered by chunk index mod 3. Register operands are reloaded for the next chunk right
// after their last use. Vector memory counters complete in issue order, so
// each wave issues its loads in the same order in the prologue as in the loop
// and never waits on a load younger than about one chunk step. The V and
// handoff pointers are not __restrict__: that keeps the compiler from moving
// prefetches across the barriers. Blocks of Ab and P above the diagonal
// (token rows 0-31, token slab 32-63) are zero and are neither loaded nor
// multiplied.
template <int DK, int DV>
__global__ __launch_bounds__(192) __attribute__((amdgpu_waves_per_eu(1, 1))) void k2_trio_kernel(
    const void* vin, const int32_t* __restrict__ cu, const int32_t* __restrict__ order,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ ckpt_base, int npairs,
    int64_t N, int H, int64_t max_chunks, const unsigned char* handoff,
    const float* __restrict__ s0, float* __restrict__ sfinal, int64_t interval,
    float* __restrict__ ckpt, int64_t ckpt_rows, PosArgs pos, float* __restrict__ o,
    float* __restrict__ sink) {
    using M = Mma<true>;
    using E = _Float16;
    using Frag = half8;
    using HO = Handoff<DK, true>;
    typedef unsigned short us8 __attribute__((ext_vector_type(8)));
    constexpr int NKS = DK / 32;  // K slabs over channels
    constexpr int NST = DK / 16;  // state row tiles
    constexpr int NRT = C / 16;   // token row tiles
    constexpr int NVB = DV / 16;  // column blocks per (seq, head)
    constexpr int kLines = (int)(HO::kBytes / 128);        // 128-byte lines per handoff block
    constexpr int kLinesWg = (kLines + NVB - 1) / NVB;     // lines each column block touches
    constexpr int NTH = (kLinesWg + 63) / 64;              // handoff touches per lane

    __shared__ __attribute__((aligned(16))) E sV[2][64][8];             // V tile B-frags [slab] (swizzled rows)
    __shared__ __attribute__((aligned(16))) f32x4 sU0[3][NRT][64];       // U0 = Ab V (result layout)
    __shared__ __attribute__((aligned(16))) float sG[3][DK];             // Gamma_last
    __shared__ __attribute__((aligned(16))) E sSU[2][NKS + 2][64][8];    // S(n) then U(n) fragments

    // wave 0 runs the chain, wave 1 the outputs, wave 2 the preparation
    const int wave = threadIdx.x >> 6;

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
    const int j0 = vb * 16;
    const int last = nch > 0 ? nch - 1 : 0;
    auto clampc = [&](int n) { return n < last ? n : last; };

    const int lane = threadIdx.x & 63;
    const int q = lane >> 4;
    const int m = lane & 15;
    const unsigned char* hbase = handoff + ((size_t)h * max_chunks + cbase) * HO::kBytes;
    auto hptr = [&](int n) { return reinterpret_cast<const E*>(hbase + (size_t)n * HO::kBytes); };
    auto chunk_len = [&](int n) {
        const int64_t left = L - (int64_t)n * C;
        return left < C ? (int)left : C;
    };
    const unsigned short* V = static_cast<const unsigned short*>(vin);

    if (wave == 0) {
        // ------------------------------------------------------ the chain ----
        Frag wn[NRT][NKS], kc[NST][2];
        auto load_w = [&](int n) {
            const E* hb = hptr(n);
#pragma unroll
            for (int r = 0; r < NRT; ++r)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) wn[r][ks] = load_frag<Frag, E>(hb + HO::kW, r * NKS + ks, lane);
        };
        auto load_k = [&](int n) {
            const E* hb = hptr(n);
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                kc[i][0] = load_frag<Frag, E>(hb + HO::kKc, i * 2 + 0, lane);
                kc[i][1] = load_frag<Frag, E>(hb + HO::kKc, i * 2 + 1, lane);
            }
        };
        // state rows owned: channel 16 i + 4 q + ii, column j0 + m
        f32x4 S[NST];
        const size_t sbase = ((size_t)seq * H + h) * DK * DV;
        if (s0) {
#pragma unroll
            for (int i = 0; i < NST; ++i)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) S[i][ii] = s0[sbase + (size_t)(16 * i + 4 * q + ii) * DV + j0 + m];
        } else {
#pragma unroll
            for (int i = 0; i < NST; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        auto store_state = [&](float* dst) {
#pragma unroll
            for (int i = 0; i < NST; ++i)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) dst[(size_t)(16 * i + 4 * q + ii) * DV + j0 + m] = S[i][ii];
        };
        // U0 (result layout) and Gamma_last rows of a chunk, read from LDS one
        // step ahead (wave 1 writes chunk n + 2 while wave 0 runs chunk n)
        f32x4 u0[NRT], gl[NST];
        auto read_prep = [&](int n) {
            const int b = n % 3;
#pragma unroll
            for (int r = 0; r < NRT; ++r) u0[r] = sU0[b][r][lane];
#pragma unroll
            for (int i = 0; i < NST; ++i) gl[i] = *reinterpret_cast<const f32x4*>(&sG[b][16 * i + 4 * q]);
        };
        auto step = [&](int n, int pn) {
            const int par = n & 1;
            // U = U0 - W S, slab by slab as S converts; S <- Gamma S meanwhile
            Frag sf[NKS];
            f32x4 U[NRT];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    sf[ks][ii] = (E)S[2 * ks][ii];
                    sf[ks][4 + ii] = (E)S[2 * ks + 1][ii];
                }
#pragma unroll
                for (int r = 0; r < NRT; ++r) U[r] = M::run(wn[r][ks], sf[ks], ks == 0 ? u0[r] : U[r]);
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) *reinterpret_cast<Frag*>(&sSU[par][ks][lane][0]) = sf[ks];
#pragma unroll
            for (int i = 0; i < NST; ++i) S[i] = S[i] * gl[i];
            __builtin_amdgcn_sched_barrier(0);
            load_w(pn);
            read_prep(n + 1);
            __builtin_amdgcn_sched_barrier(0);
            Frag uf[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    uf[s][ii] = (E)U[2 * s][ii];
                    uf[s][4 + ii] = (E)U[2 * s + 1][ii];
                }
                *reinterpret_cast<Frag*>(&sSU[par][NKS + s][lane][0]) = uf[s];
            }
            // S <- diag(Gamma_last) S + Kc^T U
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                const f32x4 a = M::run(kc[i][0], uf[0], S[i]);
                S[i] = M::run(kc[i][1], uf[1], a);
            }
            __builtin_amdgcn_sched_barrier(0);
            load_k(pn);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        load_w(0);
        load_k(0);
        __syncthreads();  // U0 and Gamma of chunks 0 and 1 ready
        __builtin_amdgcn_sched_barrier(0);
        read_prep(0);
        // Drain the prologue's loads: the compiler orders them freely, and the
        // loop's memory waits must only reflect the loop's own issue order.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        // Chunks run in segments that end on checkpoint boundaries, so the
        // chunk loop itself never branches; each checkpoint is stored between
        // segments. Without checkpoints there is one segment.
        StopWalk sw(pos, seq, L, interval, nch);
        int64_t cidx = ckpt_base ? ckpt_base[seq] : 0;
        for (int n = 0;;) {
            const int stop = sw.next();
            for (; n < stop; ++n) step(n, clampc(n + 1));
            bool stored = false;
            if (sw.take_interval(stop)) {
                if (cidx < ckpt_rows) store_state(ckpt + (cidx * H + h) * (size_t)DK * DV);
                ++cidx;
                stored = true;
            }
            for (int j; sw.take_position(stop, j);) {
                store_state(pos.states + ((size_t)j * H + h) * DK * DV);
                stored = true;
            }
            // drain the state stores here, so that the chunk loop's memory
            // waits need not allow for them (they are rare)
            if (stored) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            if (stop >= nch) break;
        }
        if (sfinal) store_state(sfinal + sbase);
    } else if (wave == 2) {
        // ------------------------------------------ next-chunk preparation ----
        // V: load instruction i covers rows 32 i + lane / 2, 16-byte half
        // lane % 2 of the row's 32-byte segment (two lanes per row)
        const int vhalf = lane & 1;
        const int glane = lane < DK / 4 ? lane : 0;  // Gamma_last: lane holds channels 4l..4l+3
        int tline[NTH];  // this lane's lines of a handoff block (clamped into the block)
#pragma unroll
        for (int k = 0; k < NTH; ++k) {
            const int t = vb * kLinesWg + (lane + 64 * k < kLinesWg ? lane + 64 * k : kLinesWg - 1);
            tline[k] = t < kLines ? t : kLines - 1;
        }
        Frag ab0[NRT], ab1[2];
        us8 vr[2];
        f32x4 gr;
        auto load_prep = [&](int n) {
            const int64_t left = L - (int64_t)n * C;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 32 * i + (lane >> 1);
                const int64_t tok = tstart + (int64_t)n * C + (r < left ? r : left - 1);
                vr[i] = *reinterpret_cast<const us8*>(V + (tok * H + h) * (int64_t)DV + j0 + 8 * vhalf);
            }
            const E* hb = hptr(n);
#pragma unroll
            for (int r = 0; r < NRT; ++r) {
                ab0[r] = load_frag<Frag, E>(hb + HO::kAb, HO::tri(r, 0), lane);
                if (r >= 2) ab1[r - 2] = load_frag<Frag, E>(hb + HO::kAb, HO::tri(r, 1), lane);
            }
            gr = *reinterpret_cast<const f32x4*>(
                reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(hb) + HO::kGlastBytes) +
                4 * glane);
        };
        // one 4-byte read in each of this column block's share of the lines of
        // chunk n's handoff block, and in this lane's V row: brings them to L2
        // V: a row of the head spans DV / 64 lines, shared by all the head's
        // column blocks; this workgroup touches every line of its own share of
        // the chunk's rows (lane i: line i % LPV of row i / LPV of the share)
        constexpr int LPV = DV / 64;                   // 128-byte lines per V row
        constexpr int VROWS = (C + NVB - 1) / NVB;     // rows this workgroup touches
        const int vt_row = vb * VROWS + (lane / LPV < VROWS ? lane / LPV : VROWS - 1);
        const int vt_line = lane % LPV;
        typedef float Touch[NTH + 1];
        auto touch = [&](int n, Touch& t) {
            const float* hb = reinterpret_cast<const float*>(hptr(n));
#pragma unroll
            for (int k = 0; k < NTH; ++k) t[k] = hb[tline[k] * 32];
            const int64_t left = L - (int64_t)n * C;
            const int r = vt_row < C ? vt_row : C - 1;
            const int64_t tok = tstart + (int64_t)n * C + (r < left ? r : left - 1);
            t[NTH] = *reinterpret_cast<const float*>(V + (tok * H + h) * (int64_t)DV + 64 * vt_line);
        };
        // V tile rows are stored XOR-swizzled (row R at R ^ (R / 16)), which
        // keeps both the scattered 2-byte writes and the fragment reads free of
        // bank conflicts.
        auto prep = [&](int n, int b) {  // into LDS buffer b
            const int len = chunk_len(n);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 32 * i + (lane >> 1);  // token
                const int w32 = r & 31;
                const int vq = (w32 & 15) >> 2, ve = (w32 & 3) + ((w32 >> 4) << 2);
                const bool valid = r < len;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const int R = 8 * vhalf + kk + 16 * vq;
                    const float x = bf16_to_f32(vr[i][kk]);
                    sV[i][R ^ vq][ve] = (E)(valid ? x : 0.f);
                }
            }
            const int rsw = lane ^ (lane >> 4);
            const Frag vf0 = *reinterpret_cast<const Frag*>(&sV[0][rsw][0]);
            const Frag vf1 = *reinterpret_cast<const Frag*>(&sV[1][rsw][0]);
#pragma unroll
            for (int r = 0; r < NRT; ++r) {
                f32x4 u = M::run(ab0[r], vf0, f32x4{0.f, 0.f, 0.f, 0.f});
                if (r >= 2) u = M::run(ab1[r - 2], vf1, u);
                sU0[b][r][lane] = u;
            }
            if (lane < DK / 4) *reinterpret_cast<f32x4*>(&sG[b][4 * lane]) = gr;
        };
        float acc = 0.f;
        Touch ta = {}, tb = {};
        auto consume = [&](const Touch& t) {
#pragma unroll
            for (int k = 0; k <= NTH; ++k) acc += t[k];
        };
        // one chunk step: prepare chunk n + 2 (loaded one step ago), load chunk
        // n + 3, consume the touches of two steps ago and touch chunk n + 5
        auto iter = [&](int n, Touch& t) {
            prep(clampc(n + 2), (n + 2) % 3);
            __builtin_amdgcn_sched_barrier(0);
            load_prep(clampc(n + 3));
            __builtin_amdgcn_sched_barrier(0);
            consume(t);
            touch(clampc(n + 5), t);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        if (nch > 0) {
            load_prep(0);
            prep(0, 0);
            load_prep(clampc(1));
            prep(clampc(1), 1);
            load_prep(clampc(2));
            touch(clampc(3), ta);
            touch(clampc(4), tb);
        }
        __syncthreads();  // U0 and Gamma of chunks 0 and 1 ready
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): as in wave 0
        int n = 0;
        for (; n + 1 < nch; n += 2) {
            iter(n, ta);
            iter(n + 1, tb);
        }
        if (n < nch) iter(n, ta);
        // keeps the touches alive; no real sum has this bit pattern (a NaN payload)
        consume(ta);
        consume(tb);
        if (__float_as_uint(acc) == 0x7fc0deadu) sink[lane] = acc;
    } else {
        // ------------------------------------------------------ outputs ----
        // a sink slot per lane and row tile: distinct addresses, so the compiler
        // keeps all four stores of a step (the memory waits count them)
        float* sink_base = sink + (size_t)(id & (kSinkSlots - 1)) * kThreads * kSinkFloats;
        Frag qd[NRT][NKS], pp0[NRT], pp1[2];
        auto load_o = [&](int n) {  // in the order the products consume them
            const E* hb = hptr(n);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int r = 0; r < NRT; ++r) qd[r][ks] = load_frag<Frag, E>(hb + HO::kQd, r * NKS + ks, lane);
#pragma unroll
            for (int r = 0; r < NRT; ++r) pp0[r] = load_frag<Frag, E>(hb + HO::kP, HO::tri(r, 0), lane);
            pp1[0] = load_frag<Frag, E>(hb + HO::kP, HO::tri(2, 1), lane);
            pp1[1] = load_frag<Frag, E>(hb + HO::kP, HO::tri(3, 1), lane);
        };
        // O(n)^T from the fragments wave 0 left at parity n & 1; lane (q, m)
        // holds token 16 r + m, columns 4q .. 4q+3. n = -1 is a dry run whose
        // stores all go to the sink (it keeps the loop free of branches).
        auto output = [&](int n, int pn) {
            const int par = n & 1;
            Frag sf[NKS], uf[2];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) sf[ks] = *reinterpret_cast<const Frag*>(&sSU[par][ks][lane][0]);
            uf[0] = *reinterpret_cast<const Frag*>(&sSU[par][NKS][lane][0]);
            uf[1] = *reinterpret_cast<const Frag*>(&sSU[par][NKS + 1][lane][0]);
            f32x4 O[NRT];
#pragma unroll
            for (int r = 0; r < NRT; ++r) O[r] = M::run(sf[0], qd[r][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int ks = 1; ks < NKS; ++ks)
#pragma unroll
                for (int r = 0; r < NRT; ++r) O[r] = M::run(sf[ks], qd[r][ks], O[r]);
#pragma unroll
            for (int r = 0; r < NRT; ++r) {
                O[r] = M::run(uf[0], pp0[r], O[r]);
                if (r >= 2) O[r] = M::run(uf[1], pp1[r - 2], O[r]);
            }
            __builtin_amdgcn_sched_barrier(0);
            load_o(pn);
            __builtin_amdgcn_sched_barrier(0);
            const int len = n < 0 ? 0 : chunk_len(n);
            const int64_t tok0 = tstart + (int64_t)n * C;
#pragma unroll
            for (int r = 0; r < NRT; ++r) {
                const int tok = 16 * r + m;
                float* op = tok < len ? o + ((tok0 + tok) * H + h) * (int64_t)DV + j0 + 4 * q
                                      : sink_base + (size_t)(64 * r + lane) * kSinkFloats;
                *reinterpret_cast<f32x4*>(op) = O[r];
            }
        };
        if (nch > 0) load_o(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): as in wave 0
        for (int n = 0; n < nch; ++n) {
            output(n - 1, n);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        }
        if (nch > 0) output(nch - 1, nch - 1);
    }
}

// Five-wave scan: one workgroup = one (sequence, head) and two column blocks
// of 16 value columns, on one CU. The rate at which a CU's vector-memory
// path takes loads (about 25 B/clk when every CU streams) bounds a scan
// step; so the operands both column blocks need (W, Kc^T; Qd, P) are
// fetched once per CU.
//   waves 0, 1  the chains of the two column blocks: U = U0 - W S, then
//               S <- diag(Gamma_last) S + Kc^T U, with S in registers and W,
//               Kc^T read from LDS one step ahead.
//   wave 2      outputs of both blocks, one chunk behind the chains:
//               O^T = S^T Qd^T + U^T P^T (Qd and P loaded once for both).
//   wave 3      preparation, two chunks ahead: V tiles, U0 = Ab V for both
//               blocks and Gamma_last into LDS.
//   wave 4      loader: W and Kc^T straight into a three-slot LDS ring three
//               chunks ahead, and touches of the lines five chunks ahead.
// One barrier per chunk. Vector memory counters complete in issue order, so
// every wave drains its prologue loads before its loop and issues each
// loop's loads in a fixed order; the V and handoff pointers are not
// __restrict__, which keeps prefetches from moving across the barriers.
// TWIN: the grid also runs a second scan over the same handoff (TwinScan:
// zero values, its own initial states, final states and outputs), its
// workgroups beside the first scan's on the same XCD, so both read each
// handoff line from that XCD's L2.
template <int DK, int DV, int NCB, bool TWIN>
__global__ __launch_bounds__(64 * (NCB + 3)) __attribute__((amdgpu_waves_per_eu(1, 2))) void k2_quad_kernel(
    const void* vin, const int32_t* __restrict__ cu, const int32_t* __restrict__ order,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ ckpt_base, int npairs,
    int64_t N, int H, int64_t max_chunks, const unsigned char* handoff,
    const float* __restrict__ s0, float* __restrict__ sfinal, int64_t interval,
    float* __restrict__ ckpt, int64_t ckpt_rows, PosArgs pos, float* __restrict__ o,
    float* __restrict__ sink, TwinScan tw) {
    using M = Mma<true>;
    using E = _Float16;
    using Frag = half8;
    using HO = Handoff<DK, true>;
    typedef unsigned short us8 __attribute__((ext_vector_type(8)));
    constexpr int NKS = DK / 32;    // K slabs over channels
    constexpr int NST = DK / 16;    // state row tiles
    constexpr int NRT = C / 16;     // token row tiles
    constexpr int NVB = DV / 16;    // column blocks per (seq, head)
    constexpr int NWG = NVB / NCB;  // workgroups per (seq, head) and scan
    constexpr int NSUB = TWIN ? 2 * NWG : NWG;  // workgroups sharing a handoff block
    constexpr int LPR = 2 * NCB;    // prep: lanes per V row segment (16 bytes each)
    constexpr int RPI = 64 / LPR;   // prep: V rows per load instruction
    constexpr int NWF = NRT * NKS;  // W fragments per chunk
    constexpr int NKF = NST * 2;    // Kc^T fragments per chunk
    constexpr int kLines = (int)(HO::kBytes / 128);       // 128-byte lines per handoff block
    constexpr int kLinesWg = (kLines + NSUB - 1) / NSUB;  // lines each workgroup touches
    static_assert(!TWIN || DK == DV, "the twin's states have the first scan's shape");
    constexpr int NTH = (kLinesWg + 63) / 64;           // handoff touches per lane

    __shared__ __attribute__((aligned(16))) E sWK[3][NWF + NKF][64][8];   // W then Kc^T fragments
    __shared__ __attribute__((aligned(16))) f32x4 sU0[3][NCB][NRT][64];      // U0 per block (result layout)
    __shared__ __attribute__((aligned(16))) float sG[3][DK];                 // Gamma_last
    __shared__ __attribute__((aligned(16))) E sSU[2][NCB][NKS + 2][64][8];   // [parity][block] S, U fragments
    __shared__ __attribute__((aligned(16))) E sV[NCB][2][64][8];             // prep: V tiles [block][slab] (swizzled rows)
    __shared__ __attribute__((aligned(16))) float sTrash[64];              // loader: target of the L2 touches

    const int id = blockIdx.x;
    const int xcd = id & 7, slot = id >> 3;
    const int pair = xcd + 8 * (slot / NSUB);
    const int sub = slot % NSUB;              // share of the handoff touches
    const bool twin = TWIN && sub >= NWG;     // a workgroup of the second scan
    const int j0 = (sub % NWG) * 16 * NCB;    // first of the workgroup's columns
    if (pair >= npairs) return;
    if (twin) {
        vin = tw.zero_v;
        s0 = tw.initial_state;
        sfinal = tw.final_state;
        o = tw.o;
    }
    // value rows: token stride H * DV, head stride DV (the twin's one zero row: 0)
    const int64_t vts = twin ? 0 : (int64_t)H * DV;
    const int64_t vhs = twin ? 0 : DV;
    const int rank = pair / H, h = pair % H;
    const int seq = order ? order[rank] : rank;
    int64_t tstart = 0, L = N;
    if (cu) seq_range(cu, seq, N, tstart, L);
    const int cbase = chunk_start ? chunk_start[seq] : 0;
    int nch = (int)((L + C - 1) / C);
    if (cbase + (int64_t)nch > max_chunks) nch = cbase < max_chunks ? (int)(max_chunks - cbase) : 0;
    const int last = nch > 0 ? nch - 1 : 0;
    auto clampc = [&](int n) { return n < last ? n : last; };

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4;
    const int m = lane & 15;
    const unsigned char* hbase = handoff + ((size_t)h * max_chunks + cbase) * HO::kBytes;
    auto hptr = [&](int n) { return reinterpret_cast<const E*>(hbase + (size_t)n * HO::kBytes); };
    auto chunk_len = [&](int n) {
        const int64_t left = L - (int64_t)n * C;
        return left < C ? (int)left : C;
    };
    const unsigned short* V = static_cast<const unsigned short*>(vin);
    // this lane's V row of chunk n (rows past the end repeat the last valid row)
    auto vrow = [&](int n) {
        const int64_t left = L - (int64_t)n * C;
        const int64_t tok = tstart + (int64_t)n * C + (lane < left ? lane : left - 1);
        return V + tok * vts + h * vhs + j0;
    };

    if (wave < NCB) {
        // ----------------------------------------------------- the chains ----
        const int cb = wave, jc = j0 + 16 * cb;
        Frag wn[NRT][NKS], kc[NST][2];
        f32x4 u0[NRT], gl[NST];
        auto read_w = [&](int n) {
            const E* b = &sWK[n % 3][0][0][0];
#pragma unroll
            for (int r = 0; r < NRT; ++r)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    wn[r][ks] = *reinterpret_cast<const Frag*>(b + ((r * NKS + ks) * 64 + lane) * 8);
        };
        auto read_k = [&](int n) {
            const E* b = &sWK[n % 3][NWF][0][0];
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                kc[i][0] = *reinterpret_cast<const Frag*>(b + ((i * 2 + 0) * 64 + lane) * 8);
                kc[i][1] = *reinterpret_cast<const Frag*>(b + ((i * 2 + 1) * 64 + lane) * 8);
            }
        };
        auto read_prep = [&](int n) {
            const int b = n % 3;
#pragma unroll
            for (int r = 0; r < NRT; ++r) u0[r] = sU0[b][cb][r][lane];
#pragma unroll
            for (int i = 0; i < NST; ++i) gl[i] = *reinterpret_cast<const f32x4*>(&sG[b][16 * i + 4 * q]);
        };
        // state rows owned: channel 16 i + 4 q + ii, column jc + m
        f32x4 S[NST];
        const size_t sbase = ((size_t)seq * H + h) * DK * DV;
        if (s0) {
#pragma unroll
            for (int i = 0; i < NST; ++i)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) S[i][ii] = s0[sbase + (size_t)(16 * i + 4 * q + ii) * DV + jc + m];
        } else {
#pragma unroll
            for (int i = 0; i < NST; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        auto store_state = [&](float* dst) {
#pragma unroll
            for (int i = 0; i < NST; ++i)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) dst[(size_t)(16 * i + 4 * q + ii) * DV + jc + m] = S[i][ii];
        };
        auto step = [&](int n) {
            const int par = n & 1;
            // U = U0 - W S, slab by slab as S converts; S <- Gamma S meanwhile
            Frag sf[NKS];
            f32x4 U[NRT];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    sf[ks][ii] = (E)S[2 * ks][ii];
                    sf[ks][4 + ii] = (E)S[2 * ks + 1][ii];
                }
#pragma unroll
                for (int r = 0; r < NRT; ++r) U[r] = M::run(wn[r][ks], sf[ks], ks == 0 ? u0[r] : U[r]);
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) *reinterpret_cast<Frag*>(&sSU[par][cb][ks][lane][0]) = sf[ks];
#pragma unroll
            for (int i = 0; i < NST; ++i) S[i] = S[i] * gl[i];
            __builtin_amdgcn_sched_barrier(0);
            read_w(n + 1);
            read_prep(n + 1);
            __builtin_amdgcn_sched_barrier(0);
            Frag uf[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    uf[s][ii] = (E)U[2 * s][ii];
                    uf[s][4 + ii] = (E)U[2 * s + 1][ii];
                }
                *reinterpret_cast<Frag*>(&sSU[par][cb][NKS + s][lane][0]) = uf[s];
            }
            // S <- diag(Gamma_last) S + Kc^T U
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                const f32x4 a = M::run(kc[i][0], uf[0], S[i]);
                S[i] = M::run(kc[i][1], uf[1], a);
            }
            __builtin_amdgcn_sched_barrier(0);
            read_k(n + 1);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        __syncthreads();  // chunks 0 and 1 staged
        __builtin_amdgcn_sched_barrier(0);
        read_w(0);
        read_k(0);
        read_prep(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loop waits only on its own loads
        // Chunks run in segments that end on checkpoint boundaries, so the
        // chunk loop itself never branches; each checkpoint is stored between
        // segments. Without checkpoints there is one segment.
        StopWalk sw(pos, seq, L, interval, nch);
        int64_t cidx = ckpt_base ? ckpt_base[seq] : 0;
        for (int n = 0;;) {
            const int stop = sw.next();
            for (; n < stop; ++n) step(n);
            bool stored = false;
            if (sw.take_interval(stop)) {
                if (cidx < ckpt_rows) store_state(ckpt + (cidx * H + h) * (size_t)DK * DV);
                ++cidx;
                stored = true;
            }
            for (int j; sw.take_position(stop, j);) {
                store_state(pos.states + ((size_t)j * H + h) * DK * DV);
                stored = true;
            }
            if (stored) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): drain the (rare) state stores
            if (stop >= nch) break;
        }
        if (sfinal) store_state(sfinal + sbase);
    } else if (wave == NCB + 2) {
        // ------------------------------------------------------- loader ----
        // W and Kc^T go global -> LDS directly (no registers), three chunks
        // ahead into the ring slot the chains finished with one step ago.
        // Before each barrier the loader waits only for the chunk the chains
        // read next (issued one step earlier), so later loads stay in flight.
        // It touches no LDS itself: the compiler would drain every load in
        // flight before such an access.
        typedef __attribute__((address_space(3))) void* lds_ptr;
        int tline[NTH];
#pragma unroll
        for (int k = 0; k < NTH; ++k) {
            const int t = sub * kLinesWg + (lane + 64 * k < kLinesWg ? lane + 64 * k : kLinesWg - 1);
            tline[k] = t < kLines ? t : kLines - 1;
        }
        auto dma_wk = [&](int n) {
            const E* hb = hptr(n);
            const int bf = n % 3;
#pragma unroll
            for (int f = 0; f < NWF; ++f)
                __builtin_amdgcn_global_load_lds((const void*)(hb + HO::kW + ((size_t)f * 64 + lane) * 8),
                                                 (lds_ptr)&sWK[bf][f][0][0], 16, 0, 0);
#pragma unroll
            for (int f = 0; f < NKF; ++f)
                __builtin_amdgcn_global_load_lds((const void*)(hb + HO::kKc + ((size_t)f * 64 + lane) * 8),
                                                 (lds_ptr)&sWK[bf][NWF + f][0][0], 16, 0, 0);
        };
        // one 4-byte read in each of this workgroup's share of the lines of
        // chunk n's handoff block and in this lane's V row: brings them to L2.
        // The touches load into an LDS area nobody reads, so no register has
        // to wait for them.
        auto touch = [&](int n) {
            const float* hb = reinterpret_cast<const float*>(hptr(n));
#pragma unroll
            for (int k = 0; k < NTH; ++k)
                __builtin_amdgcn_global_load_lds((const void*)(hb + tline[k] * 32), (lds_ptr)&sTrash[0], 4, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)vrow(n), (lds_ptr)&sTrash[0], 4, 0, 0);
        };
        // Per step, in this order: the DMA (NWF + NKF) and the touches
        // (NTH + 1). The DMA of chunk n + 2 (issued one step ago) has completed
        // once at most kAfter later operations remain outstanding.
        constexpr int kAfter = (NTH + 1) + (NWF + NKF) + (NTH + 1);
        static_assert(kAfter <= 63, "the memory counter field holds at most 63");
        auto bar = [&]() {  // barrier without the compiler's full memory drain
            __builtin_amdgcn_s_waitcnt(0x0F70 | (kAfter & 15) | ((kAfter >> 4) << 14));  // vmcnt(kAfter)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        if (nch > 0) {
            dma_wk(0);
            dma_wk(clampc(1));
            dma_wk(clampc(2));
            touch(clampc(3));
            touch(clampc(4));
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): chunks 0-2 complete
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // chunks 0 and 1 staged
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        for (int n = 0; n < nch; ++n) {
            // DMA chunk n + 3, touch chunk n + 5
            dma_wk(clampc(n + 3));
            __builtin_amdgcn_sched_barrier(0);
            touch(clampc(n + 5));
            __builtin_amdgcn_sched_barrier(0);
            bar();
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    } else if (wave == NCB + 1) {
        // -------------------------------------------------- preparation ----
        const int glane = lane < DK / 4 ? lane : 0;  // Gamma_last: lane holds channels 4l..4l+3
        // V: instruction i loads rows RPI i + lane / LPR, 16-byte piece
        // lane % LPR of the workgroup's row segment (coalesced)
        const int vpiece = lane % LPR;
        Frag ab0[NRT], ab1[2];
        us8 vr[LPR];
        f32x4 gr;
        auto load_prep = [&](int n) {
            const int64_t left = L - (int64_t)n * C;
#pragma unroll
            for (int i = 0; i < LPR; ++i) {
                const int r = RPI * i + lane / LPR;
                const int64_t tok = tstart + (int64_t)n * C + (r < left ? r : left - 1);
                vr[i] = *reinterpret_cast<const us8*>(V + tok * vts + h * vhs + j0 + 8 * vpiece);
            }
            const E* hb = hptr(n);
#pragma unroll
            for (int r = 0; r < NRT; ++r) {
                ab0[r] = load_frag<Frag, E>(hb + HO::kAb, HO::tri(r, 0), lane);
                if (r >= 2) ab1[r - 2] = load_frag<Frag, E>(hb + HO::kAb, HO::tri(r, 1), lane);
            }
            gr = *reinterpret_cast<const f32x4*>(
                reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(hb) + HO::kGlastBytes) +
                4 * glane);
        };
        // V tile rows are stored XOR-swizzled (row R of block b at R ^ (R / 16 | 4 b)),
        // which keeps both the scattered 2-byte writes and the fragment reads
        // free of bank conflicts.
        auto prep = [&](int n) {  // V tiles, U0 = Ab V of both blocks and Gamma_last into buffer n mod 3
            const int bf = n % 3;
            const int len = chunk_len(n);
#pragma unroll
            for (int i = 0; i < LPR; ++i) {
                const int r = RPI * i + lane / LPR;  // token
                const int slab = r >> 5, w32 = r & 31;
                const int vq = (w32 & 15) >> 2, ve = (w32 & 3) + ((w32 >> 4) << 2);
                const int bk = vpiece >> 1;
                const bool valid = r < len;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int c = 8 * (vpiece & 1) + k;
                    const int R = c + 16 * vq;
                    const float x = bf16_to_f32(vr[i][k]);
                    sV[bk][slab][R ^ (vq | (bk << 2))][ve] = (E)(valid ? x : 0.f);
                }
            }
            const int rsw = lane ^ (lane >> 4);
#pragma unroll
            for (int bk = 0; bk < NCB; ++bk) {
                const Frag vf0 = *reinterpret_cast<const Frag*>(&sV[bk][0][rsw ^ (bk << 2)][0]);
                const Frag vf1 = *reinterpret_cast<const Frag*>(&sV[bk][1][rsw ^ (bk << 2)][0]);
#pragma unroll
                for (int r = 0; r < NRT; ++r) {
                    f32x4 u = M::run(ab0[r], vf0, f32x4{0.f, 0.f, 0.f, 0.f});
                    if (r >= 2) u = M::run(ab1[r - 2], vf1, u);
                    sU0[bf][bk][r][lane] = u;
                }
            }
            if (lane < DK / 4) *reinterpret_cast<f32x4*>(&sG[bf][4 * lane]) = gr;
        };
        if (nch > 0) {
            load_prep(0);
            prep(0);
            load_prep(clampc(1));
            prep(clampc(1));
            load_prep(clampc(2));
        }
        __syncthreads();  // chunks 0 and 1 staged
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): as in the chains
        for (int n = 0; n < nch; ++n) {
            // stage chunk n + 2 (loaded one step ago), load chunk n + 3
            prep(clampc(n + 2));
            __builtin_amdgcn_sched_barrier(0);
            load_prep(clampc(n + 3));
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        // ------------------------------------------------------ outputs ----
        // a sink slot per lane, row tile and block: distinct addresses, so the
        // compiler keeps every store of a step (the memory waits count them)
        float* sink_base = sink + (size_t)(id & (kSinkSlots - 1)) * kThreads * kSinkFloats;
        Frag qd[NRT][NKS], pp0[NRT], pp1[2];
        auto load_o = [&](int n) {  // in the order the products consume them
            const E* hb = hptr(n);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int r = 0; r < NRT; ++r) qd[r][ks] = load_frag<Frag, E>(hb + HO::kQd, r * NKS + ks, lane);
#pragma unroll
            for (int r = 0; r < NRT; ++r) pp0[r] = load_frag<Frag, E>(hb + HO::kP, HO::tri(r, 0), lane);
            pp1[0] = load_frag<Frag, E>(hb + HO::kP, HO::tri(2, 1), lane);
            pp1[1] = load_frag<Frag, E>(hb + HO::kP, HO::tri(3, 1), lane);
        };
        // O(n)^T of both blocks from the fragments the chains left at parity
        // n & 1; lane (q, m) holds token 16 r + m, columns 4q .. 4q+3. n = -1
        // is a dry run whose stores all go to the sink (no branch in the loop).
        auto output = [&](int n, int pn) {
            const int par = n & 1;
            f32x4 O[NCB][NRT];
#pragma unroll
            for (int b = 0; b < NCB; ++b) {
                Frag sf[NKS], uf[2];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) sf[ks] = *reinterpret_cast<const Frag*>(&sSU[par][b][ks][lane][0]);
                uf[0] = *reinterpret_cast<const Frag*>(&sSU[par][b][NKS][lane][0]);
                uf[1] = *reinterpret_cast<const Frag*>(&sSU[par][b][NKS + 1][lane][0]);
#pragma unroll
                for (int r = 0; r < NRT; ++r) O[b][r] = M::run(sf[0], qd[r][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int ks = 1; ks < NKS; ++ks)
#pragma unroll
                    for (int r = 0; r < NRT; ++r) O[b][r] = M::run(sf[ks], qd[r][ks], O[b][r]);
#pragma unroll
                for (int r = 0; r < NRT; ++r) {
                    O[b][r] = M::run(uf[0], pp0[r], O[b][r]);
                    if (r >= 2) O[b][r] = M::run(uf[1], pp1[r - 2], O[b][r]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            load_o(pn);
            __builtin_amdgcn_sched_barrier(0);
            const int len = n < 0 ? 0 : chunk_len(n);
            const int64_t tok0 = tstart + (int64_t)n * C;
#pragma unroll
            for (int b = 0; b < NCB; ++b)
#pragma unroll
                for (int r = 0; r < NRT; ++r) {
                    const int tok = 16 * r + m;
                    float* op = tok < len ? o + ((tok0 + tok) * H + h) * (int64_t)DV + j0 + 16 * b + 4 * q
                                          : sink_base + (size_t)(64 * r + lane) * kSinkFloats + 4 * b;
                    *reinterpret_cast<f32x4*>(op) = O[b][r];
                }
        };
        if (nch > 0) load_o(0);
        __syncthreads();  // chunks 0 and 1 staged
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): as in the chains
        for (int n = 0; n < nch; ++n) {
            output(n - 1, n);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        }
        if (nch > 0) output(nch - 1, nch - 1);
    }
}

// ---------------------------------------------------- position advance ----
// States at arbitrary positions with bf16 inputs. The scan stored the state
// S_n at the start of the chunk that holds position P; the first r = P mod 64
// rows of that chunk advance it in chunk form on the matrix cores, from the
// handoff K1 wrote for the chunk (rows < r of Ab and W involve only rows < r):
//   U_r = rows < r of (Ab V - W S_n),
//   S_P = Diag(e^{G_{r-1}}) S_n + Kc_r^T U_r,
//   Kc_r[s][c] = k_s[c] e^{G_{r-1}[c] - G_s[c]} for s < r, 0 otherwise,
// G the cumulative decay from the chunk start (the same chunk algebra as the
// scan step, stopped after r rows). Kc_r is formed here from k and g: the
// handoff's Kc is relative to the chunk end. One workgroup per (position,
// head, 64 value columns), one 16-column tile per wave; operands as in the
// scan (fp16, fp32 accumulation), S_n rounded to fp16 where it enters W S_n.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void advance_chunk_kernel(
    const void* __restrict__ kin, const void* __restrict__ vin, const float* __restrict__ g,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_start, int num_seqs,
    int64_t N, int H, int64_t max_chunks, const unsigned char* __restrict__ handoff, PosArgs pos,
    unsigned front) {
    using M = Mma<true>;
    using E = _Float16;
    using Frag = half8;
    using HO = Handoff<DK, true>;
    constexpr int NKS = DK / 32;  // 32-wide channel slabs
    constexpr int NRT = DK / 16;  // 16-row channel tiles
    constexpr int CT = DV / 16;   // value-column tiles
    constexpr int KP = DK + 4;
    constexpr int NQ = kThreads / DK;  // row groups of the cumulative sum
    constexpr int RPQ = C / NQ;
    constexpr int SP = DV + 4;
    __shared__ __attribute__((aligned(16))) float sG[C][KP];  // G * log2(e); rows >= r: G_{r-1}
    __shared__ __attribute__((aligned(16))) float sK[C][KP];  // keys (normalised with L2); rows >= r: 0
    __shared__ __attribute__((aligned(16))) float sS[DK][SP];  // S_n
    __shared__ double sTot[NQ][DK];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int q = lane >> 4, m = lane & 15;
    constexpr int NCH = (CT + 3) / 4;  // workgroups per (position, head): 64 columns each
    const int half = (int)(blockIdx.x % (unsigned)NCH);
    const int jh = (int)(blockIdx.x / (unsigned)NCH);
    const int j = jh / H, h = jh % H;
    int seq = 0;
    int64_t st = 0, L = N;
    if (cu) {  // sequence of position j: the last s with offsets[s] <= j
        int lo = 0, hi = num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pos.offsets[mid] <= j) lo = mid;
            else hi = mid - 1;
        }
        seq = lo;
        seq_range(cu, seq, N, st, L);
    }
    int64_t P = pos.values[j];
    P = P < 0 ? 0 : (P > L ? L : P);
    const int r = (int)(P % C);
    if (r == 0) return;  // the scan stored the exact state
    const int64_t ci = (cu ? (int64_t)chunk_start[seq] : 0) + (P - r) / C;
    const int64_t t0 = st + (P - r);
    const E* hb = reinterpret_cast<const E*>(handoff + ((size_t)h * max_chunks + ci) * HO::kBytes);
    float* S = pos.states + ((size_t)j * H + h) * (size_t)(DK * DV);

    // this workgroup's 64 columns of S_n into LDS (16-byte loads, all issued
    // before the decay and key work; the other column half belongs to another
    // workgroup, which updates it in place)
    constexpr int WC = DV < 64 ? DV : 64;  // columns per workgroup
    constexpr int SV = DK * WC / 4 / kThreads;
    f32x4 sreg[SV];
#pragma unroll
    for (int u = 0; u < SV; ++u) {
        const int i = t + u * kThreads;
        sreg[u] = *reinterpret_cast<const f32x4*>(S + (size_t)(i / (WC / 4)) * DV + WC * half + 4 * (i % (WC / 4)));
    }
#pragma unroll
    for (int u = 0; u < SV; ++u) {
        const int i = t + u * kThreads;
        *reinterpret_cast<f32x4*>(&sS[i / (WC / 4)][WC * half + 4 * (i % (WC / 4))]) = sreg[u];
    }

    // ---- cumulative decay over rows < r (rows >= r add 0) and keys: g
    // floored and summed in fp64 as in K1, stored as fp32 G * log2(e)
    {
        const int c = t % DK, grp = t / DK;
        float gl[RPQ];
#pragma unroll
        for (int i = 0; i < RPQ; ++i) {
            const int row = grp * RPQ + i;
            float x = row < r ? g[((t0 + row) * H + h) * DK + c] : 0.f;
            if ((front & kFrontGate) && row < r) x = -__expf(x);
            gl[i] = fmaxf(x, -kGFloorBF16);
        }
        double acc = 0;
#pragma unroll
        for (int i = 0; i < RPQ; ++i) acc += (double)gl[i];
        sTot[grp][c] = acc;
        __syncthreads();
        double run = 0;
        for (int p = 0; p < grp; ++p) run += sTot[p][c];
#pragma unroll
        for (int i = 0; i < RPQ; ++i) {
            run += (double)gl[i];
            sG[grp * RPQ + i][c] = (float)(run * 1.4426950408889634);
        }
    }
    {  // keys: four threads per row, DK / 4 channels each, 16-byte loads
        const int row = t >> 2, part = t & 3;
        constexpr int NC = DK / 4;
        const u16x8* src = reinterpret_cast<const u16x8*>(
            static_cast<const unsigned short*>(kin) + ((t0 + (row < r ? row : 0)) * H + h) * DK + part * NC);
        u16x8 raw[NC / 8];
#pragma unroll
        for (int v8 = 0; v8 < NC / 8; ++v8) raw[v8] = src[v8];
        float kv[NC];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            kv[e] = row < r ? bf16_to_f32(raw[e / 8][e % 8]) : 0.f;
            ss += kv[e] * kv[e];
        }
        if (front & kFrontL2) {
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            const float inv = 1.f / sqrtf(ss + kL2Eps);
#pragma unroll
            for (int e = 0; e < NC; ++e) kv[e] *= inv;
        }
#pragma unroll
        for (int e = 0; e < NC; ++e) sK[row][part * NC + e] = kv[e];
    }
    __syncthreads();

    // Kc_r as A operands: rows = channels 16 ct + m, K = tokens of slab ts (permuted)
    Frag kc[NRT][2];
#pragma unroll
    for (int ct = 0; ct < NRT; ++ct) {
        const int c = 16 * ct + m;
        const float gr = sG[r - 1][c];
#pragma unroll
        for (int ts = 0; ts < 2; ++ts)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sr = 32 * ts + perm32(q, e);
                kc[ct][ts][e] = (E)(sK[sr][c] * fast_exp2(gr - sG[sr][c]));
            }
    }

    // Ab and -W operands: the same for every column tile, loaded once per wave
    Frag abf[4][2], wnf[4][NKS];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int ts = 0; ts < 2; ++ts)  // token slab 1 of row tiles 0-1 is zero (not stored)
            abf[rt][ts] = (ts == 0 || rt >= 2) ? load_frag<Frag, E>(hb + HO::kAb, HO::tri(rt, ts), lane) : Frag{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) wnf[rt][ks] = load_frag<Frag, E>(hb + HO::kW, rt * NKS + ks, lane);
    }

    {
        const int ctile = 4 * half + wave;
        if (ctile >= CT) return;  // DV = 64 uses one workgroup of four tiles
        const int col = 16 * ctile + m;
        // B operands: S_n (K = channels) and V (K = tokens, rows clamped into the sequence data)
        Frag sb[NKS], vb[2];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) sb[ks][e] = (E)sS[32 * ks + perm32(q, e)][col];
#pragma unroll
        for (int ts = 0; ts < 2; ++ts)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                int64_t row = t0 + 32 * ts + perm32(q, e);
                row = row < N ? row : N - 1;
                vb[ts][e] = (E)bf16_to_f32(static_cast<const unsigned short*>(vin)[(row * H + h) * DV + col]);
            }
        f32x4 old[NRT];  // S_n at this lane's result rows
#pragma unroll
        for (int ct = 0; ct < NRT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) old[ct][i] = sS[16 * ct + 4 * q + i][col];
        // U = Ab V + (-W) S_n, row tiles of tokens
        f32x4 u[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ts = 0; ts < 2; ++ts) acc = M::run(abf[rt][ts], vb[ts], acc);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) acc = M::run(wnf[rt][ks], sb[ks], acc);
            u[rt] = acc;
        }
        // two stacked U tiles are the B operand of one token slab
        Frag ub[2];
#pragma unroll
        for (int ts = 0; ts < 2; ++ts)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ub[ts][i] = (E)u[2 * ts][i];
                ub[ts][4 + i] = (E)u[2 * ts + 1][i];
            }
#pragma unroll
        for (int ct = 0; ct < NRT; ++ct) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ts = 0; ts < 2; ++ts) acc = M::run(kc[ct][ts], ub[ts], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 16 * ct + 4 * q + i;
                S[(size_t)c * DV + col] = fast_exp2(sG[r - 1][c]) * old[ct][i] + acc[i];
            }
        }
    }
}

// ------------------------------------------------------------- host side ---
struct Plan {
    int32_t* chunk_start;
    int32_t* ckpt_base;
    int32_t* order;
    unsigned char* handoff;
    float* sink;
    int64_t max_chunks;
};

Plan make_plan(const PrefillArgs& a) {
    Plan p;
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    p.chunk_start = reinterpret_cast<int32_t*>(ws);
    p.ckpt_base = p.chunk_start + (a.num_seqs + 1);
    p.order = p.ckpt_base + (a.num_seqs + 1);
    p.handoff = ws + table_bytes(a.num_seqs);
    p.sink = reinterpret_cast<float*>(p.handoff - kSinkBytes);
    p.max_chunks = max_chunks(a.total_tokens, a.num_seqs);
    return p;
}

template <int DK, int DV, int NT, bool BF16>
void launch_scan(const PrefillArgs& a, const Plan& p, int npairs, hipStream_t stream) {
    constexpr int NVB = DV / (16 * NT);
    const bool varlen = a.cu_seqlens != nullptr;
    const int64_t groups = (npairs + 7) / 8;
    const unsigned grid = (unsigned)(groups * 8 * NVB);
    hipLaunchKernelGGL((k2_scan_kernel<DK, DV, NT, BF16>), dim3(grid), dim3(kThreads), 0, stream,
                       a.v, a.cu_seqlens, varlen ? p.order : nullptr,
                       varlen ? p.chunk_start : nullptr, varlen ? p.ckpt_base : nullptr, npairs,
                       a.total_tokens, a.H, p.max_chunks, p.handoff, a.initial_state, a.final_state,
                       a.ckpt_interval, a.ckpt_states, a.ckpt_rows, a.pos, a.o, p.sink);
}

// Three-wave scan: one workgroup per (pair, 16 columns). When there are no
// more such workgroups than CUs, each asks for enough (unused) LDS that no two
// share a CU, so they spread out instead of queueing on one CU's vector
// memory path.
template <int DK, int DV>
void launch_trio(const PrefillArgs& a, const Plan& p, int npairs, int cus, int lds_max,
                 hipStream_t stream) {
    constexpr int NVB = DV / 16;  // workgroups per (seq, head)
    const bool varlen = a.cu_seqlens != nullptr;
    const int64_t groups = (npairs + 7) / 8;
    const unsigned grid = (unsigned)(groups * 8 * NVB);
    const int64_t wgs = (int64_t)npairs * NVB;
    const int64_t per_cu = (wgs + cus - 1) / cus;
    unsigned pad = 0;
    // the kernel's static LDS, asked once per process
    static const int64_t have = [] {
        hipFuncAttributes fa;
        return hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(&k2_trio_kernel<DK, DV>)) == hipSuccess
                   ? (int64_t)fa.sharedSizeBytes
                   : (int64_t)-1;
    }();
    if (per_cu < 2 && have >= 0) {
        const int64_t want = (int64_t)lds_max / per_cu - 512;
        pad = want > have ? (unsigned)(want - have) : 0u;
    }
    hipLaunchKernelGGL((k2_trio_kernel<DK, DV>), dim3(grid), dim3(192), pad, stream,
                       a.v, a.cu_seqlens, varlen ? p.order : nullptr,
                       varlen ? p.chunk_start : nullptr, varlen ? p.ckpt_base : nullptr, npairs,
                       a.total_tokens, a.H, p.max_chunks, p.handoff, a.initial_state, a.final_state,
                       a.ckpt_interval, a.ckpt_states, a.ckpt_rows, a.pos, a.o, p.sink);
}

// Five-wave scan: one workgroup per (pair, 32 columns), one per CU (its LDS
// use, about 150 KB, keeps a second one off the CU).
template <int DK, int DV, int NCB, bool TWIN>
void launch_quad(const PrefillArgs& a, const Plan& p, int npairs, hipStream_t stream) {
    constexpr int NWG = DV / (16 * NCB) * (TWIN ? 2 : 1);
    const bool varlen = a.cu_seqlens != nullptr;
    const int64_t groups = (npairs + 7) / 8;
    const unsigned grid = (unsigned)(groups * 8 * NWG);
    hipLaunchKernelGGL((k2_quad_kernel<DK, DV, NCB, TWIN>), dim3(grid), dim3(64 * (NCB + 3)), 0, stream,
                       a.v, a.cu_seqlens, varlen ? p.order : nullptr,
                       varlen ? p.chunk_start : nullptr, varlen ? p.ckpt_base : nullptr, npairs,
                       a.total_tokens, a.H, p.max_chunks, p.handoff, a.initial_state, a.final_state,
                       a.ckpt_interval, a.ckpt_states, a.ckpt_rows, a.pos, a.o, p.sink, a.twin);
}

// Chunk-step times on MI355X (D = 128, us x 100) the scan choice works with.
constexpr int64_t kStepTrio = 135, kStepQuad = 158, kStepNt4 = 308;

// The least (rounds of workgroups over the CUs) x (step time) over the bf16
// scans for `blocks` 16-column blocks of one scan.
int64_t bf16_scan_cost(int64_t blocks, int Dv, int cus, int* which) {
    auto rounds = [&](int64_t wgs) { return (wgs + cus - 1) / cus; };
    const int64_t trio = rounds(blocks) * kStepTrio, quad = rounds((blocks + 1) / 2) * kStepQuad;
    const int64_t nt4 = Dv % 64 == 0 ? rounds((blocks + 3) / 4) * kStepNt4 : INT64_MAX;
    const int w = trio <= quad && trio <= nt4 ? 0 : (quad <= nt4 ? 1 : 2);
    if (which) *which = w;
    return w == 0 ? trio : (w == 1 ? quad : nt4);
}

template <int DK, int DV, bool BF16>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
    const Plan p = make_plan(a);
    const bool varlen = a.cu_seqlens != nullptr;
    const bool prepare = (a.phases & 1u) != 0, scan = (a.phases & 2u) != 0;
    if (prepare && varlen && !a.schedule_ready)
        hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(kPrepThreads), 0, stream, a.cu_seqlens, a.num_seqs,
                           a.total_tokens, a.ckpt_interval, p.chunk_start, p.ckpt_base, p.order);
    if (prepare && p.max_chunks > 0 && a.total_tokens > 0) {
        auto k1 = (a.frontend & kFrontL2) ? &k1_prep_kernel<DK, BF16, true>
                                          : &k1_prep_kernel<DK, BF16, false>;
        hipLaunchKernelGGL(k1, dim3((unsigned)(p.max_chunks * a.H)), dim3(kThreads), 0, stream,
                           a.q, a.k, a.g, a.beta, a.cu_seqlens, varlen ? p.chunk_start : nullptr,
                           a.num_seqs, a.total_tokens, a.H, p.max_chunks, a.frontend, p.handoff);
    }
    // Scan design. Every scan workgroup streams the whole handoff of its
    // (sequence, head) through its CU, about 62 KB per chunk for D = 128, and
    // the rate at which a CU's vector-memory path takes those loads (about
    // 25 B/clk when every CU streams) bounds each chunk step. Chunk-step
    // times on MI355X (D = 128) when this rule was set: three-wave kernel,
    // one 16-column block per CU: 1.35 us (1.2 now); five-wave kernel, two
    // blocks sharing a CU's operand stream: 1.58 us; four-wave kernel with 64
    // columns: 3.08 us (with 16 or 32 columns, 1.73 and 2.11 us: never the
    // best choice). Pick (bf16_scan_cost, kStep* above)
    // the least (rounds of workgroups over the CUs) x (step time): few
    // (sequence, head) pairs take the three-wave kernel, a few times more the
    // five-wave one, thousands the 64-column one. fp32 operands take the
    // four-wave kernel with 16 columns.
    const int npairs = a.num_seqs * a.H;
    const DeviceInfo di = device_info();
    const int cus = di.cus, lds_max = di.lds_per_block;
    enum { kTrio, kQuad, kNt4, kNt1 } design = kNt1;
    if (BF16) {
        int w = 0;
        bf16_scan_cost((int64_t)npairs * (DV / 16), DV, cus, &w);
        design = w == 0 ? kTrio : (w == 1 ? kQuad : kNt4);
    }
    if (scan && a.twin.zero_v) {  // both scans in one five-wave launch
        if constexpr (BF16 && DK == DV) {
            if (a.ckpt_interval != 0 || a.pos.num_pos != 0) return hipErrorInvalidValue;
            launch_quad<DK, DV, 2, true>(a, p, npairs, stream);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (scan) {
        switch (design) {
            case kTrio: launch_trio<DK, DV>(a, p, npairs, cus, lds_max, stream); break;
            case kQuad: launch_quad<DK, DV, 2, false>(a, p, npairs, stream); break;
            case kNt4:  // bf16 only (fp32 inputs always take the 16-column kernel)
                if constexpr (BF16) launch_scan<DK, DV, 4, BF16>(a, p, npairs, stream);
                break;
            default: launch_scan<DK, DV, 1, BF16>(a, p, npairs, stream); break;
        }
        if (a.pos.num_pos > 0) {  // finish the states of positions inside a chunk
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            if (!BF16) return launch_advance(a, stream);  // fp32 inputs: token by token
            hipLaunchKernelGGL((advance_chunk_kernel<DK, DV>), dim3((unsigned)((int64_t)a.pos.num_pos * a.H * (DV / 64))),
                               dim3(kThreads), 0, stream, a.k, a.v, a.g, a.cu_seqlens,
                               varlen ? p.chunk_start : nullptr, a.num_seqs, a.total_tokens, a.H,
                               p.max_chunks, p.handoff, a.pos, a.frontend);
        }
    }
    return hipGetLastError();
}

}  // namespace

bool prefill_twin_scan_pays(int npairs, int Dk, int Dv, bool bf16, int cus) {
    if (!bf16 || Dk != Dv || npairs <= 0 || cus <= 0) return false;
    const int64_t blocks = (int64_t)npairs * (Dv / 16);
    // one launch: the five-wave scan over both scans' blocks (two per workgroup)
    const int64_t both = ((blocks + cus - 1) / cus) * kStepQuad;
    return both < 2 * bf16_scan_cost(blocks, Dv, cus, nullptr);
}

size_t prefill_workspace_bytes(int64_t total_tokens, int num_seqs, int H, int Dk, int Dv,
                               bool bf16) {
    (void)Dv;
    return table_bytes(num_seqs) +
           (size_t)H * (size_t)max_chunks(total_tokens, num_seqs) * handoff_bytes(Dk, bf16);
}

hipError_t launch_prefill_plain(const PrefillArgs& a, hipStream_t stream) {
    const bool b = a.bf16;
    if (a.Dk == 128 && a.Dv == 128) return b ? launch_typed<128, 128, true>(a, stream) : launch_typed<128, 128, false>(a, stream);
    if (a.Dk == 128 && a.Dv == 64) return b ? launch_typed<128, 64, true>(a, stream) : launch_typed<128, 64, false>(a, stream);
    if (a.Dk == 64 && a.Dv == 128) return b ? launch_typed<64, 128, true>(a, stream) : launch_typed<64, 128, false>(a, stream);
    if (a.Dk == 64 && a.Dv == 64) return b ? launch_typed<64, 64, true>(a, stream) : launch_typed<64, 64, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
