// spec_verify.hip -- CDNA4 (gfx950) kernels and C ABI of the batched
// verify-and-sample step of speculative decoding.
//
// Sources (page title, section):
//   [FI] "Fast Inference from Transformers via Speculative Decoding" (paper
//        summary page): "Standardized Sampling"; "Speculative Sampling: The
//        Core Algorithm", Algorithm 1 Phases 3 and 4.
//   [PB] "Speculative Decoding Paper Breakdown: Lossless Draft-and-Verify
//        Acceleration for Autoregressive Transformers": section 3, "The
//        Algorithm at Position i"; "Reference Implementation" (q <= 0 accepts).
//   [ST] "The exact decoding shortcut that burns compute when guesses miss":
//        correction_distribution (target row when the residual mass <= 1e-15).
//
// Three launches per call (two in greedy mode), all on the caller's stream:
//
//   1. row stage (k_rows_sample / k_rows_greedy).  The grid enumerates
//      (position k, sequence b, chunk c) with k slowest.  A workgroup streams
//      one chunk of target row (b, k) with 128-bit loads and reduces it to a
//      partial (max, sum of exp) -- or (max, first argmax) in greedy mode --
//      and the last workgroup of a row (arrival counter) merges the row's
//      partials and takes the acceptance decision for position k, setting
//      bit k of the sequence's reject mask on a rejection.  A workgroup that
//      finds an earlier position of its sequence already rejected skips its
//      chunk: rows past the first rejection are never needed ([FI] Phase 3,
//      the walk stops at the first rejection), so with position-major launch
//      order most of them are never read.  The decision at each position is
//      independent of the others, so skipping changes no result.
//
//   2. draw stage (k_draw_sums + k_draw_finish, or k_draw_greedy).  n is the
//      index of the lowest set bit of the reject mask (gamma if none).  For
//      every sequence the row n of the target (and of the draft, when
//      n < gamma) is streamed in chunks; each workgroup computes, in double
//      precision, e_v = exp((z_v - max)/T) and the chunk sums needed for the
//      residual mass.  Then one workgroup per sequence turns them into the
//      exact row normaliser, picks the chunk holding the inverse-CDF target
//      and scans it to find the token.
//
// Numerics.  The row stage uses fp32 exp2 with a two-term log2(e)/T and a
// per-chunk correction of the rounded shift, and accumulates in fp64; the
// acceptance threshold is formed in fp64.  The draw stage works entirely in
// fp64 (e_v, normaliser, residual, prefix sums), so its token boundaries
// agree with an fp64 evaluation to rounding level.
//
// Workspace: reject masks and arrival counters, then scratch for partials
// and per-row statistics.  It must be all zero before a call, and each
// consumer clears what it read, so a finished call leaves all of it zero
// again -- whatever shape the next call has.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint64_t kInvalidBit = 1ull << 63;
constexpr double kResidEps = 1e-15;  // [ST] correction_distribution
constexpr double kLog2e = 1.4426950408889634073599246810018921;

// Elements per thread of one row-stage chunk (a chunk is 32 KiB of input).
constexpr int kEptBf16 = 64;
constexpr int kEptFp32 = 32;
constexpr int kChunkBf16 = kEptBf16 * kThreads;  // 16384 elements
constexpr int kChunkFp32 = kEptFp32 * kThreads;  // 8192 elements
// Elements per thread of one draw-stage chunk (a chunk is 8192 elements).
constexpr int kEpt2 = 32;
constexpr int kChunk2 = kEpt2 * kThreads;

// Per-row statistics written by the row stage, read by the draw stage.
struct RowStat {
    float m;       // row max of the raw logits
    int32_t amax;  // greedy: first index attaining m
    double S;      // sum_v exp((z_v - m)/T)
    double P;      // p_k(x_k)
    double Q;      // q_k(x_k)
};
static_assert(sizeof(RowStat) == 32, "RowStat layout");

// Per-chunk partial of the draw stage.
struct DrawPart {
    double E;   // sum of e_v over the chunk
    double EA;  // sum of e_v over {v : p_v > q_v} (residual support)
    double QA;  // sum of q_v over the same set
    double pad;
};
static_assert(sizeof(DrawPart) == 32, "DrawPart layout");

struct Layout {
    size_t mask_off, cnt1_off, control_bytes;
    size_t part1_off, stats_off, part2_off, total;
    int nch1_max, nch2_max;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout make_layout(int B, int gamma, int V)
{
    Layout L;
    const size_t rows = (size_t)B * (size_t)(gamma + 1);
    L.nch1_max = (V + kChunkFp32 - 1) / kChunkFp32;
    L.nch2_max = (V + kChunk2 - 1) / kChunk2;
    size_t off = 0;
    L.mask_off = off;  off = align256(off + sizeof(uint64_t) * (size_t)B);
    L.cnt1_off = off;  off = align256(off + sizeof(uint64_t) * rows);
    L.control_bytes = off;
    L.part1_off = off; off = align256(off + 2 * sizeof(uint64_t) * rows * (size_t)L.nch1_max);
    L.stats_off = off; off = align256(off + sizeof(RowStat) * rows);
    L.part2_off = off; off = align256(off + sizeof(DrawPart) * (size_t)B * (size_t)L.nch2_max);
    L.total = off;
    return L;
}

// ------------------------------------------------------------------ device helpers

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p)
{
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishes a block's partial result for the last block of its row or
// sequence.  Each word goes out with a device-scope atomic exchange, and the
// exchanged-out old values feed the operand of the caller's arrival-counter
// increment, so every exchange has completed device-wide before the count
// that reveals it can be observed.  The last block reads the words back with
// device-scope atomic loads.  (A release/acquire pair at agent scope orders
// the same thing but writes back the whole L2 on every block, about ten times
// the cost of the streaming work itself.)  `zero` is a kernel argument that
// is always 0 and opaque to the compiler; the result is always 0.
template <int N>
__device__ __forceinline__ uint32_t publish(uint64_t* slot, const uint64_t (&w)[N], uint32_t zero)
{
    uint64_t dep = 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
        dep ^= __hip_atomic_exchange(slot + i, w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (uint32_t)(dep ^ (dep >> 32)) & zero;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DT>
__device__ __forceinline__ float load_one(const void* base, int64_t idx)
{
    if constexpr (DT == SV_FP32) {
        return static_cast<const float*>(base)[idx];
    } else {
        return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[idx]) << 16);
    }
}

__device__ __forceinline__ float load_one_rt(const void* base, int dt, int64_t idx)
{
    return dt == SV_FP32 ? load_one<SV_FP32>(base, idx) : load_one<SV_BF16>(base, idx);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ int wave_max_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ int wave_min_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    return v;
}

// Block reductions over kThreads threads; every thread gets the result.
// `sm` must hold kWaves entries and is free again on return.
__device__ float block_max(float v, float* sm)
{
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sm[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = fmaxf(r, sm[w]);
    __syncthreads();
    return r;
}
__device__ double block_sum(double v, double* sm)
{
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = sm[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r += sm[w];
    __syncthreads();
    return r;
}
__device__ int block_max_i(int v, int* sm)
{
    v = wave_max_i(v);
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = sm[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = max(r, sm[w]);
    __syncthreads();
    return r;
}
__device__ int block_min_i(int v, int* sm)
{
    v = wave_min_i(v);
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = sm[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = min(r, sm[w]);
    __syncthreads();
    return r;
}

// Exclusive prefix sum over the block (thread order); also returns the total.
__device__ double block_exclusive_scan(double v, double* sm, double* total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    double incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        double t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) sm[wid] = incl;
    __syncthreads();
    double base = 0.0, tot = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < wid) base += sm[w];
        tot += sm[w];
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// Argmax pairs: larger value wins, ties go to the lower index.
__device__ __forceinline__ void amax_merge(float& v, int& i, float v2, int i2)
{
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
__device__ __forceinline__ void wave_amax(float& v, int& i)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float v2 = __shfl_xor(v, o, 64);
        int i2 = __shfl_xor(i, o, 64);
        amax_merge(v, i, v2, i2);
    }
}
__device__ void block_amax(float& v, int& i, float* smf, int* smi)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float v2 = __shfl_xor(v, o, 64);
        int i2 = __shfl_xor(i, o, 64);
        amax_merge(v, i, v2, i2);
    }
    if ((threadIdx.x & 63) == 0) { smf[threadIdx.x >> 6] = v; smi[threadIdx.x >> 6] = i; }
    __syncthreads();
    v = smf[0]; i = smi[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) amax_merge(v, i, smf[w], smi[w]);
    __syncthreads();
}

// 2^a in double for a <= 0, relative error below 2e-14: a = k + f with k
// the nearest integer (rounded by adding 1.5 * 2^52, which leaves k in the
// low word) and |f| <= 1/2; 2^f by a degree-9 polynomial interpolating it at
// Chebyshev nodes of [-1/2, 1/2]; 2^k applied with ldexp, which rounds to a
// subnormal or to 0 below the normal range.  a is clamped at -1100 first, so
// -inf (and NaN) give exactly 0.  The coefficients travel as kernel
// arguments: uniform values stay in scalar registers, which fp64 FMAs read
// directly (as literals they would be rebuilt in vector registers for every
// element).
struct Exp2Coef {
    double c[10];  // c[0] multiplies f^9, c[9] is the constant term
    double magic;  // 1.5 * 2^52
    double lo;     // clamp: -1100
};
constexpr Exp2Coef kExp2Coef = {{1.0208789509527192e-07, 1.3259656070717964e-06, 1.5252656913569549e-05,
                                 0.00015403433688494325, 0.0013333558230514875, 0.009618129194063072,
                                 0.05550410866444786, 0.24022650695639422, 0.6931471805599502,
                                 1.0000000000000138},
                                6755399441055744.0, -1100.0};

__device__ __forceinline__ double exp2_f64(double a, const Exp2Coef& k)
{
    a = fmax(a, k.lo);
    const double t = a + k.magic;
    const double f = a - (t - k.magic);
    const int n = __double2loint(t);
    double p = k.c[0];
#pragma unroll
    for (int i = 1; i < 10; ++i) p = fma(f, p, k.c[i]);
    return ldexp(p, n);
}

// Loads this thread's share of one row-stage chunk into registers.  Vector
// path: 128-bit loads, consecutive threads on consecutive 16-byte pieces
// (requires a 16-byte aligned row start and V a multiple of the vector
// width); all loads are issued before any value is used.  Scalar path: one
// element per load, consecutive threads on consecutive elements.  Elements
// past V read as -inf; a chunk that ends past V clamps its addresses to the
// row instead of branching per load.  Element e of x sits at index:
//   vector: v0 + (j * kThreads + tid) * W + (e % W), j = e / W
//   scalar: v0 + e * kThreads + tid
template <int DT, bool VEC, int EPT, bool FULL>
__device__ __forceinline__ void load_chunk_impl(const void* rowp, int v0, int V, float (&x)[EPT])
{
    const int tid = threadIdx.x;
    if constexpr (VEC) {
        constexpr int W = DT == SV_BF16 ? 8 : 4;
        constexpr int NV = EPT / W;
        constexpr size_t ES = DT == SV_BF16 ? 2 : 4;
        uint4 raw[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            int idx = v0 + (j * kThreads + tid) * W;
            if constexpr (!FULL) idx = min(idx, V - W);
            raw[j] = *reinterpret_cast<const uint4*>(static_cast<const char*>(rowp) + (size_t)idx * ES);
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            uint4 w = raw[j];
            if constexpr (!FULL) {
                if (v0 + (j * kThreads + tid) * W >= V) {
                    const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
                    w = make_uint4(ninf, ninf, ninf, ninf);
                }
            }
            if constexpr (DT == SV_BF16) {
                x[j * 8 + 0] = bf16_lo(w.x); x[j * 8 + 1] = bf16_hi(w.x);
                x[j * 8 + 2] = bf16_lo(w.y); x[j * 8 + 3] = bf16_hi(w.y);
                x[j * 8 + 4] = bf16_lo(w.z); x[j * 8 + 5] = bf16_hi(w.z);
                x[j * 8 + 6] = bf16_lo(w.w); x[j * 8 + 7] = bf16_hi(w.w);
            } else {
                x[j * 4 + 0] = __uint_as_float(w.x); x[j * 4 + 1] = __uint_as_float(w.y);
                x[j * 4 + 2] = __uint_as_float(w.z); x[j * 4 + 3] = __uint_as_float(w.w);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int idx = v0 + e * kThreads + tid;
            if constexpr (FULL) {
                x[e] = load_one<DT>(rowp, idx);
            } else {
                const float z = load_one<DT>(rowp, min(idx, V - 1));
                x[e] = idx < V ? z : -INFINITY;
            }
        }
    }
}

template <int DT, bool VEC, int EPT>
__device__ __forceinline__ void load_chunk(const void* rowp, int v0, int V, float (&x)[EPT])
{
    if (v0 + EPT * kThreads <= V) load_chunk_impl<DT, VEC, EPT, true>(rowp, v0, V, x);
    else load_chunk_impl<DT, VEC, EPT, false>(rowp, v0, V, x);
}

// This thread's share of one row-stage chunk, kept as loaded: raw 128-bit
// words on the vector path (bf16 values are unpacked at each use, which
// costs one integer op and halves the registers), floats otherwise.
// get8(g, z) yields elements 8g .. 8g+7 in the order of load_chunk.
template <int DT, bool VEC, int EPT>
struct ChunkRegs {
    static constexpr int W = DT == SV_BF16 ? 8 : 4;
    uint4 raw[EPT / W];
    __device__ __forceinline__ void load(const void* rowp, int v0, int V)
    {
        if (v0 + EPT * kThreads <= V) load_impl<true>(rowp, v0, V);
        else load_impl<false>(rowp, v0, V);
    }
    template <bool FULL>
    __device__ __forceinline__ void load_impl(const void* rowp, int v0, int V)
    {
        constexpr size_t ES = DT == SV_BF16 ? 2 : 4;
        const int tid = threadIdx.x;
#pragma unroll
        for (int j = 0; j < EPT / W; ++j) {
            int idx = v0 + (j * kThreads + tid) * W;
            if constexpr (!FULL) idx = min(idx, V - W);
            raw[j] = *reinterpret_cast<const uint4*>(static_cast<const char*>(rowp) + (size_t)idx * ES);
        }
        if constexpr (!FULL) {
            const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
#pragma unroll
            for (int j = 0; j < EPT / W; ++j)
                if (v0 + (j * kThreads + tid) * W >= V) raw[j] = make_uint4(ninf, ninf, ninf, ninf);
        }
    }
    // Hides the loaded words from the optimizer, so values unpacked before
    // this point are recomputed after it rather than kept live (the raw
    // words take half the registers).
    __device__ __forceinline__ void opaque()
    {
#pragma unroll
        for (int j = 0; j < EPT / W; ++j) asm volatile("" : "+v"(raw[j].x), "+v"(raw[j].y), "+v"(raw[j].z), "+v"(raw[j].w));
    }
    __device__ __forceinline__ void get8(int g, float (&z)[8]) const
    {
        if constexpr (DT == SV_BF16) {
            const uint4 w = raw[g];
            z[0] = bf16_lo(w.x); z[1] = bf16_hi(w.x); z[2] = bf16_lo(w.y); z[3] = bf16_hi(w.y);
            z[4] = bf16_lo(w.z); z[5] = bf16_hi(w.z); z[6] = bf16_lo(w.w); z[7] = bf16_hi(w.w);
        } else {
            const uint4 a = raw[2 * g], b = raw[2 * g + 1];
            z[0] = __uint_as_float(a.x); z[1] = __uint_as_float(a.y); z[2] = __uint_as_float(a.z); z[3] = __uint_as_float(a.w);
            z[4] = __uint_as_float(b.x); z[5] = __uint_as_float(b.y); z[6] = __uint_as_float(b.z); z[7] = __uint_as_float(b.w);
        }
    }
};
template <int DT, int EPT>
struct ChunkRegs<DT, false, EPT> {
    float x[EPT];
    __device__ __forceinline__ void load(const void* rowp, int v0, int V) { load_chunk<DT, false, EPT>(rowp, v0, V, x); }
    __device__ __forceinline__ void opaque() {}
    __device__ __forceinline__ void get8(int g, float (&z)[8]) const
    {
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = x[g * 8 + e];
    }
};

template <bool VEC, int EPT, int W>
__device__ __forceinline__ int elem_index(int v0, int e)
{
    if constexpr (VEC) return v0 + ((e / W) * kThreads + (int)threadIdx.x) * W + (e % W);
    else return v0 + e * kThreads + (int)threadIdx.x;
}

struct RowParams {
    const void* logits;
    const void* probs;
    const int32_t* tokens;
    const float* uniforms;
    uint64_t* mask;
    uint64_t* cnt1;   // per row: arrivals (low 16 bits), rejection evidence (high 48)
    uint64_t* part1;  // [rows][nch][2]
    RowStat* stats;
    int B, gamma, V, nch, probs_dtype;
    uint32_t zero;     // always 0 (see publish)
    float c_hi, c_lo;  // log2(e)/T split into two fp32 terms, c_lo > 0
    double cd;         // log2(e)/T in double
    Exp2Coef ex;       // kExp2Coef
};

// Shared prologue: is this (row, chunk) still needed?  Thread 0 reads the
// sequence's reject mask once and broadcasts, so the whole block agrees.
__device__ __forceinline__ bool chunk_skipped(const RowParams& p, int b, int k, int* sm_flag)
{
    if (k == 0) return false;  // position 0 is always needed (k is uniform)
    if (threadIdx.x == 0) {
        const uint64_t m = ld_agent(&p.mask[b]);
        const uint64_t earlier = k == 0 ? 0ull : (m & ((1ull << k) - 1ull));
        *sm_flag = ((m & kInvalidBit) | earlier) ? 1 : 0;
    }
    __syncthreads();
    return *sm_flag != 0;
}

// Shared epilogue, run by wave 0 alone once the block's reductions are done
// (the other waves have left; no block barrier follows): count this block in
// and learn whether it is the last block of the row; the last block resets
// the counter to zero.  Blocks that skip their chunk never count in, so a row
// with a skipped chunk has no last block (it is not needed: an earlier
// position was rejected); the draw stage clears such a row's counter and
// partial slots.
//
// The counter word also gathers evidence of a rejection (sample mode): each
// block adds, in its high 48 bits, floor(2^30 min(2, u Q s')) where s' is its
// chunk's sum of exp((z_v - z_x)/T) (z_x the draft token's logit).  Every
// term is positive, so once the running total exceeds 2^30 (plus a margin
// far above the rounding of these terms) u Q sum_v exp((z_v - z_x)/T) > 1,
// i.e. p(x) / q(x) < u: the position is rejected whatever the other chunks
// hold.  The block that sees this sets the reject bit at once, so later
// positions of the sequence stop being fetched sooner; the last block still
// takes the full decision, which is the same.
constexpr int kCountBits = 16;
constexpr uint64_t kCountMask = (1ull << kCountBits) - 1ull;
constexpr double kEvidenceScale = 0x1p30;
constexpr uint64_t kEvidenceThreshold = (1ull << 30) + (1ull << 14);

__device__ __forceinline__ uint64_t rejection_evidence(double u, double Q, double s, float mx, float zx, double cd,
                                                       const Exp2Coef& ex)
{
    if (!(Q > 0.0) || !(mx > -INFINITY)) return 0;
    const double x = zx > -INFINITY ? u * Q * s * exp2_f64(((double)mx - (double)zx) * cd, ex) : 2.0;
    return (uint64_t)(fmin(x, 2.0) * kEvidenceScale);
}

__device__ __forceinline__ bool row_arrive(const RowParams& p, int64_t row, int b, uint64_t evidence,
                                          uint64_t early_bit, uint32_t dep)
{
    uint32_t last = 0;
    if (threadIdx.x == 0) {
        const uint64_t add = 1ull + (evidence << kCountBits) + dep;
        const uint64_t old = __hip_atomic_fetch_add(&p.cnt1[row], add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = (old & kCountMask) + 1ull == (uint64_t)p.nch ? 1u : 0u;
        if (last) {
            __hip_atomic_store(&p.cnt1[row], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (early_bit && (old >> kCountBits) + evidence > kEvidenceThreshold) {
            __hip_atomic_fetch_or(&p.mask[b], early_bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    return __builtin_amdgcn_readfirstlane(last) != 0u;
}

// ----------------------------------------------------------------- row stage, sample

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_rows_sample(const RowParams p)
{
    constexpr int EPT = DT == SV_BF16 ? kEptBf16 : kEptFp32;
    constexpr int CH = EPT * kThreads;
    const int c = (int)(blockIdx.x % (unsigned)p.nch);
    const int t = (int)(blockIdx.x / (unsigned)p.nch);
    const int b = t % p.B;
    const int k = t / p.B;
    const int G1 = p.gamma + 1;
    const int64_t row = (int64_t)b * G1 + k;

    __shared__ float sm_f[kWaves];
    __shared__ double sm_d[kWaves];
    __shared__ int sm_flag;

    if (chunk_skipped(p, b, k, &sm_flag)) return;
    // The decision inputs (draft token, its logit and draft probability, the
    // uniform) are fetched while the chunk streams, in case this block turns
    // out to be the row's last.
    int xk = 0;
    float zx = 0.0f, qx = 0.0f, uk = 0.0f;
    if (threadIdx.x == 0 && k < p.gamma) {
        xk = p.tokens[(int64_t)b * p.gamma + k];
        uk = p.uniforms[(int64_t)b * G1 + k];
        if (xk >= 0 && xk < p.V) {
            zx = load_one_rt(p.logits, DT, row * p.V + xk);
            qx = load_one_rt(p.probs, p.probs_dtype, ((int64_t)b * p.gamma + k) * p.V + xk);
        }
    }
    uint32_t dep = 0;
    uint64_t evidence = 0, early_bit = 0;
    {
        const int v0 = c * CH;
        const void* rowp = static_cast<const char*>(p.logits) + (size_t)row * (size_t)p.V * (DT == SV_BF16 ? 2 : 4);
        ChunkRegs<DT, VEC, EPT> x;
        x.load(rowp, v0, p.V);

        float mx = -INFINITY;
#pragma unroll
        for (int g = 0; g < EPT / 8; ++g) {
            float z[8];
            x.get8(g, z);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, z[e]);
        }
        mx = block_max(mx, sm_f);
        x.opaque();

        double s = 0.0;
        double mc = 0.0;
        float K = 0.0f;
        if (mx > -INFINITY) {
            // exponent of element z: z*c_hi + K + z*c_lo = (z - mx)*log2(e)/T + eta,
            // with eta = K + mx*cd the rounding of the shift (corrected below).
            mc = (double)mx * p.cd;
            K = (float)(-mc);
            double acc = 0.0;
#pragma unroll
            for (int g = 0; g < EPT / 8; ++g) {
                float z[8], e8[8];
                x.get8(g, z);
#pragma unroll
                for (int e = 0; e < 8; ++e) e8[e] = __builtin_amdgcn_exp2f(fmaf(z[e], p.c_lo, fmaf(z[e], p.c_hi, K)));
                acc += (double)(((e8[0] + e8[1]) + (e8[2] + e8[3])) + ((e8[4] + e8[5]) + (e8[6] + e8[7])));
            }
            s = block_sum(acc, sm_d);
        }
        if (threadIdx.x >= 64) return;  // only wave 0 goes on (no block barrier below)
        if (threadIdx.x == 0) {
            if (mx > -INFINITY) s *= exp2(-((double)K + mc));
            const uint64_t w[2] = {(uint64_t)__float_as_uint(mx), (uint64_t)__double_as_longlong(s)};
            dep = publish(p.part1 + 2 * ((size_t)row * p.nch + c), w, p.zero);
            if (k < p.gamma && xk >= 0 && xk < p.V) {
                evidence = rejection_evidence((double)uk, (double)qx, s, mx, zx, p.cd, p.ex);
                early_bit = 1ull << k;
            }
        }
    }

    if (!row_arrive(p, row, b, evidence, early_bit, dep)) return;

    // Last block of a fully processed row: wave 0 merges the chunk partials.
    const int lane = (int)threadIdx.x;
    float M = -INFINITY;
    for (int j = lane; j < p.nch; j += 64) {
        const uint64_t* slot = p.part1 + 2 * ((size_t)row * p.nch + j);
        M = fmaxf(M, __uint_as_float((uint32_t)ld_agent(slot)));
    }
    M = wave_max(M);
    double S = 0.0;
    for (int j = lane; j < p.nch; j += 64) {
        const uint64_t* slot = p.part1 + 2 * ((size_t)row * p.nch + j);
        const float mj = __uint_as_float((uint32_t)ld_agent(slot));
        const double sj = __longlong_as_double((long long)ld_agent(slot + 1));
        if (mj > -INFINITY) S += sj * exp2_f64(((double)mj - (double)M) * p.cd, p.ex);
    }
    S = wave_sum(S);

    if (threadIdx.x == 0) {
        RowStat st;
        st.m = M;
        st.amax = -1;
        st.S = S;
        st.P = NAN;
        st.Q = NAN;
        if (k < p.gamma) {
            // [FI] Phase 3 / [PB] section 3: accept x_k iff u_k <= min(1, p/q),
            // q <= 0 accepts ([PB] Reference Implementation).
            if (xk < 0 || xk >= p.V) {
                __hip_atomic_fetch_or(&p.mask[b], kInvalidBit | (1ull << k), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            } else {
                const double P = exp2(((double)zx - (double)M) * p.cd) / S;
                const double Q = (double)qx;
                const double thr = Q <= 0.0 ? 1.0 : fmin(1.0, P / Q);
                const double u = (double)uk;
                st.P = P;
                st.Q = Q;
                if (!(u <= thr))
                    __hip_atomic_fetch_or(&p.mask[b], 1ull << k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        p.stats[row] = st;
    }
}

// ----------------------------------------------------------------- row stage, greedy

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_rows_greedy(const RowParams p)
{
    constexpr int EPT = DT == SV_BF16 ? kEptBf16 : kEptFp32;
    constexpr int W = DT == SV_BF16 ? 8 : 4;
    constexpr int CH = EPT * kThreads;
    const int c = (int)(blockIdx.x % (unsigned)p.nch);
    const int t = (int)(blockIdx.x / (unsigned)p.nch);
    const int b = t % p.B;
    const int k = t / p.B;
    const int G1 = p.gamma + 1;
    const int64_t row = (int64_t)b * G1 + k;

    __shared__ float sm_f[kWaves];
    __shared__ int sm_i[kWaves];
    __shared__ int sm_flag;

    if (chunk_skipped(p, b, k, &sm_flag)) return;
    // the draft token and its logit, for an early rejection by this chunk
    int xk = -1;
    float zx = 0.0f;
    if (threadIdx.x == 0 && k < p.gamma) {
        xk = p.tokens[(int64_t)b * p.gamma + k];
        if (xk >= 0 && xk < p.V) zx = load_one_rt(p.logits, DT, row * p.V + xk);
    }
    uint32_t dep = 0;
    {
        const int v0 = c * CH;
        const void* rowp = static_cast<const char*>(p.logits) + (size_t)row * (size_t)p.V * (DT == SV_BF16 ? 2 : 4);
        float x[EPT];
        load_chunk<DT, VEC, EPT>(rowp, v0, p.V, x);
        float bv = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int idx = elem_index<VEC, EPT, W>(v0, e);
            if (idx < p.V) amax_merge(bv, bi, x[e], idx);
        }
        block_amax(bv, bi, sm_f, sm_i);
        if (threadIdx.x >= 64) return;  // only wave 0 goes on (no block barrier below)
        if (threadIdx.x == 0) {
            const uint64_t w[1] = {((uint64_t)(uint32_t)bi << 32) | (uint64_t)__float_as_uint(bv)};
            dep = publish(p.part1 + 2 * ((size_t)row * p.nch + c), w, p.zero);
            // an element of this chunk beats the draft token for the argmax
            // (larger, or equal at a lower index): the position is rejected
            if (k < p.gamma && xk >= 0 && xk < p.V && bi != INT_MAX && (bv > zx || (bv == zx && bi < xk)))
                __hip_atomic_fetch_or(&p.mask[b], 1ull << k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    if (!row_arrive(p, row, b, 0, 0, dep)) return;

    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int j = (int)threadIdx.x; j < p.nch; j += 64) {
        const uint64_t w = ld_agent(p.part1 + 2 * ((size_t)row * p.nch + j));
        amax_merge(bv, bi, __uint_as_float((uint32_t)w), (int)(uint32_t)(w >> 32));
    }
    wave_amax(bv, bi);
    if (threadIdx.x == 0) {
        RowStat st;
        st.m = bv;
        st.amax = bi;
        st.S = NAN;
        st.P = NAN;
        st.Q = NAN;
        if (k < p.gamma) {
            // [FI] "Standardized Sampling", argmax case: the draft survives iff
            // it is the target argmax.
            const int x = p.tokens[(int64_t)b * p.gamma + k];
            uint64_t bits = 0;
            if (x < 0 || x >= p.V) bits = kInvalidBit | (1ull << k);
            else if (x != bi) bits = 1ull << k;
            if (bits) __hip_atomic_fetch_or(&p.mask[b], bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        p.stats[row] = st;
    }
}

// ------------------------------------------------------------------- draw stage

struct DrawParams {
    const void* logits;
    const void* probs;
    const int32_t* tokens;
    const float* uniforms;
    uint64_t* mask;
    uint64_t* cnt1;   // row-stage counters and partial slots, cleared per sequence
    uint64_t* part1;
    int nch1;
    RowStat* stats;
    DrawPart* part2;  // [B][nch2]
    int32_t* n_out;
    int32_t* tok_out;
    double* aux_p;
    double* aux_q;
    double* aux_resid;
    float* aux_rmax;
    double* aux_rsum;
    int B, gamma, V, nch2;
    uint32_t zero;  // always 0 (see publish)
    double cd;
    Exp2Coef ex;  // kExp2Coef
};

// Per-position values the finish of a sequence needs, loaded early by thread
// i (= position i <= gamma; gamma + 1 <= kThreads): the draft token x_i and
// the statistics of row i.
struct PosInfo {
    int32_t tok;
    RowStat st;
};
__device__ __forceinline__ PosInfo load_pos_info(const DrawParams& p, int b)
{
    PosInfo pi;
    pi.tok = 0;
    pi.st = RowStat{0.0f, 0, 0.0, 0.0, 0.0};
    const int i = threadIdx.x;
    if (i <= p.gamma) {
        pi.st = p.stats[(int64_t)b * (p.gamma + 1) + i];
        if (i < p.gamma) pi.tok = p.tokens[(int64_t)b * p.gamma + i];
    }
    return pi;
}

// Writes the per-sequence outputs and telemetry, and clears what the call
// left in the workspace for this sequence.  Called by the whole block.
__device__ void finish_sequence(const DrawParams& p, int b, int n, int t, bool invalid, double Z, bool sample,
                                const PosInfo& pi)
{
    const int G1 = p.gamma + 1;
    const int i = threadIdx.x;
    if (i < G1) {
        int32_t o;
        if (invalid) o = -1;
        else if (i < n) o = pi.tok;
        else if (i == n) o = t;
        else o = -1;
        p.tok_out[(int64_t)b * G1 + i] = o;
        const RowStat& st = pi.st;
        p.stats[(int64_t)b * G1 + i] = RowStat{0.0f, 0, 0.0, 0.0, 0.0};  // leave the workspace zero
        const bool row_seen = !invalid && i <= n;
        if (p.aux_rmax) p.aux_rmax[(int64_t)b * G1 + i] = row_seen ? st.m : NAN;
        if (p.aux_rsum) p.aux_rsum[(int64_t)b * G1 + i] = (row_seen && sample) ? st.S : NAN;
        if (i < p.gamma) {
            const bool tested = sample && row_seen;
            if (p.aux_p) p.aux_p[(int64_t)b * p.gamma + i] = tested ? st.P : NAN;
            if (p.aux_q) p.aux_q[(int64_t)b * p.gamma + i] = tested ? st.Q : NAN;
        }
    }
    // rows whose chunks were partly skipped kept their arrival count and
    // partials: clear every row-stage slot of this sequence
    for (int j = threadIdx.x; j < G1 * p.nch1; j += kThreads) {
        uint64_t* slot = p.part1 + 2 * ((size_t)b * G1 * p.nch1 + j);
        st_agent(slot, 0ull);
        st_agent(slot + 1, 0ull);
    }
    for (int i = threadIdx.x; i < G1; i += kThreads)
        __hip_atomic_store(&p.cnt1[(int64_t)b * G1 + i], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) {
        p.n_out[b] = invalid ? -1 : n;
        if (p.aux_resid) p.aux_resid[b] = (!invalid && sample && n < p.gamma) ? Z : NAN;
        p.mask[b] = 0ull;
    }
}

__device__ __forceinline__ void clear_draw_partials(const DrawParams& p, int b)
{
    for (int j = threadIdx.x; j < p.nch2; j += kThreads) p.part2[(size_t)b * p.nch2 + j] = DrawPart{0.0, 0.0, 0.0, 0.0};
}

// Any draft token of sequence b outside [0, V)?  (Checked over all gamma
// tokens, also those past the first rejection.)  Called by the whole block.
__device__ bool tokens_invalid(const DrawParams& p, const PosInfo& pi, int* sm_i)
{
    const int i = threadIdx.x;
    const int bad = (i < p.gamma && (pi.tok < 0 || pi.tok >= p.V)) ? 1 : 0;
    return block_max_i(bad, sm_i) != 0;
}

// Loads 8 consecutive elements starting at idx (a multiple of 8 on the
// vector path).  Past-the-end elements read as `pad`.
template <int DT, bool VEC, bool FULL>
__device__ __forceinline__ void load8(const void* rowp, int idx, int V, float pad, float* out)
{
    constexpr size_t ES = DT == SV_BF16 ? 2 : 4;
    if constexpr (VEC) {
        const int ci = FULL ? idx : min(idx, V - 8);
        const char* ptr = static_cast<const char*>(rowp) + (size_t)ci * ES;
        if constexpr (DT == SV_BF16) {
            const uint4 w = *reinterpret_cast<const uint4*>(ptr);
            out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x); out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
            out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z); out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
        } else {
            const uint4 a = *reinterpret_cast<const uint4*>(ptr);
            const uint4 b = *reinterpret_cast<const uint4*>(ptr + 16);
            out[0] = __uint_as_float(a.x); out[1] = __uint_as_float(a.y);
            out[2] = __uint_as_float(a.z); out[3] = __uint_as_float(a.w);
            out[4] = __uint_as_float(b.x); out[5] = __uint_as_float(b.y);
            out[6] = __uint_as_float(b.z); out[7] = __uint_as_float(b.w);
        }
        if constexpr (!FULL) {
            if (idx >= V) {
#pragma unroll
                for (int e = 0; e < 8; ++e) out[e] = pad;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = idx + e;
            if constexpr (FULL) {
                out[e] = load_one<DT>(rowp, i);
            } else {
                const float v = load_one<DT>(rowp, min(i, V - 1));
                out[e] = i < V ? v : pad;
            }
        }
    }
}

// 8 consecutive elements as raw 128-bit words (one for bf16, two for fp32).
struct Raw8 {
    uint4 a, b;
};
template <int DT, bool FULL>
__device__ __forceinline__ Raw8 load_raw8(const void* rowp, int idx, int V)
{
    constexpr size_t ES = DT == SV_BF16 ? 2 : 4;
    const int ci = FULL ? idx : min(idx, V - 8);
    const char* ptr = static_cast<const char*>(rowp) + (size_t)ci * ES;
    Raw8 r;
    r.a = *reinterpret_cast<const uint4*>(ptr);
    if constexpr (DT == SV_FP32) r.b = *reinterpret_cast<const uint4*>(ptr + 16);
    else r.b = make_uint4(0u, 0u, 0u, 0u);
    return r;
}
template <int DT>
__device__ __forceinline__ float raw8_elem(const Raw8& r, int e)
{
    if constexpr (DT == SV_BF16) {
        const uint32_t w = e < 2 ? r.a.x : e < 4 ? r.a.y : e < 6 ? r.a.z : r.a.w;
        return (e & 1) ? bf16_hi(w) : bf16_lo(w);
    } else {
        const uint32_t w = e == 0 ? r.a.x : e == 1 ? r.a.y : e == 2 ? r.a.z : e == 3 ? r.a.w
                         : e == 4 ? r.b.x : e == 5 ? r.b.y : e == 6 ? r.b.z : r.b.w;
        return __uint_as_float(w);
    }
}

// Chunk sums of the draw stage for this thread's kEpt2 elements: groups of 8
// consecutive elements at v0 + (g * kThreads + tid) * 8.  Every load of the
// chunk is issued before the arithmetic starts.
template <int DT, int PT, bool VEC, bool FULL>
__device__ __forceinline__ void draw_chunk_sums(const DrawParams& p, const void* zrow, const void* qrow,
                                                bool resid, int v0, double nMcd, double S_row,
                                                double& E, double& EA, double& QA)
{
    constexpr int NG = kEpt2 / 8;
    const int tid = (int)threadIdx.x;
    // e_v = 2^((z - M) log2(e)/T); the shift -M log2(e)/T is rounded once for
    // the whole row, a common factor that cancels in every ratio used
    auto element = [&](float zf, float qf) {
        const double e = exp2_f64(fma((double)zf, p.cd, nMcd), p.ex);
        E += e;
        if (resid) {
            const double qd = (double)qf;
            const double in = e > qd * S_row ? 1.0 : 0.0;  // in the residual support
            EA = fma(e, in, EA);
            QA = fma(qd, in, QA);
        }
    };
    if constexpr (VEC) {
        Raw8 zr[NG], qr[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) zr[g] = load_raw8<DT, FULL>(zrow, v0 + (g * kThreads + tid) * 8, p.V);
        if (resid) {
#pragma unroll
            for (int g = 0; g < NG; ++g) qr[g] = load_raw8<PT, FULL>(qrow, v0 + (g * kThreads + tid) * 8, p.V);
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int idx = v0 + (g * kThreads + tid) * 8;
            if (!FULL && idx >= p.V) continue;
#pragma unroll
            for (int e = 0; e < 8; ++e) element(raw8_elem<DT>(zr[g], e), resid ? raw8_elem<PT>(qr[g], e) : 0.0f);
        }
    } else {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int idx = v0 + (g * kThreads + tid) * 8;
            float z[8], q[8];
            load8<DT, false, FULL>(zrow, idx, p.V, -INFINITY, z);
            if (resid) load8<PT, false, FULL>(qrow, idx, p.V, 0.0f, q);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (FULL || idx + e < p.V) element(z[e], resid ? q[e] : 0.0f);
        }
    }
}

// Weight of one element of row n for the inverse-CDF draw: max(0, p - q)
// with p = e / S, or e itself for the bonus / fallback draw.
__device__ __forceinline__ double draw_weight(const DrawParams& p, bool use_resid, float z, float q, double nMcd,
                                              double invS)
{
    const double e = exp2_f64(fma((double)z, p.cd, nMcd), p.ex);
    return use_resid ? fmax(0.0, e * invS - (double)q) : e;
}

// This thread's share of one draw-stage chunk of row n (and of the draft
// row): group g holds the 8 elements from base + (g * kThreads + tid) * 8.
// Vector path: raw 128-bit words, all loads issued together; otherwise
// unpacked floats.  Elements past V must be ignored by the caller.
template <int DT, int PT, bool VEC>
struct ChunkBuf {
    static constexpr int NG = kEpt2 / 8;
    Raw8 zr[NG], qr[NG];
    __device__ __forceinline__ void load(const DrawParams& p, const void* zrow, const void* qrow, bool with_q, int base)
    {
        const int tid = (int)threadIdx.x;
#pragma unroll
        for (int g = 0; g < NG; ++g) zr[g] = load_raw8<DT, false>(zrow, base + (g * kThreads + tid) * 8, p.V);
        if (with_q) {
#pragma unroll
            for (int g = 0; g < NG; ++g) qr[g] = load_raw8<PT, false>(qrow, base + (g * kThreads + tid) * 8, p.V);
        }
    }
    __device__ __forceinline__ float z(int g, int e) const { return raw8_elem<DT>(zr[g], e); }
    __device__ __forceinline__ float q(int g, int e) const { return raw8_elem<PT>(qr[g], e); }
};
template <int DT, int PT>
struct ChunkBuf<DT, PT, false> {
    static constexpr int NG = kEpt2 / 8;
    float zv[NG][8], qv[NG][8];
    __device__ __forceinline__ void load(const DrawParams& p, const void* zrow, const void* qrow, bool with_q, int base)
    {
        const int tid = (int)threadIdx.x;
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = min(base + (g * kThreads + tid) * 8 + e, p.V - 1);
                zv[g][e] = load_one<DT>(zrow, i);
                qv[g][e] = with_q ? load_one<PT>(qrow, i) : 0.0f;
            }
    }
    __device__ __forceinline__ float z(int g, int e) const { return zv[g][e]; }
    __device__ __forceinline__ float q(int g, int e) const { return qv[g][e]; }
};

// Where the draw of sequence b reads: n from the reject mask, row n of the
// target (and of the draft when n < gamma), and the row stage's statistics.
struct SeqDraw {
    int n;
    bool resid;         // n < gamma: residual draw, else bonus draw
    bool invalid_seen;  // the row stage met an out-of-range draft token
    const void* zrow;
    const void* qrow;
    double nMcd;        // -max_v z * log2(e)/T, rounded once for the row
    double S_row;       // the row stage's normaliser (fp32 exponentials)
};
template <int DT, int PT>
__device__ __forceinline__ SeqDraw seq_draw(const DrawParams& p, int b)
{
    SeqDraw sd;
    const uint64_t m = p.mask[b];
    const uint64_t rej = m & ((1ull << p.gamma) - 1ull);
    sd.invalid_seen = (m & kInvalidBit) != 0;
    sd.n = rej ? __builtin_ctzll(rej) : p.gamma;
    sd.resid = sd.n < p.gamma;
    const int64_t row = (int64_t)b * (p.gamma + 1) + sd.n;
    const RowStat st = p.stats[row];  // in bounds for any mask (n <= gamma)
    sd.nMcd = -(double)st.m * p.cd;
    sd.S_row = st.S;
    sd.zrow = static_cast<const char*>(p.logits) + (size_t)row * p.V * (DT == SV_BF16 ? 2 : 4);
    sd.qrow = sd.resid ? static_cast<const char*>(p.probs) +
                             (size_t)((int64_t)b * p.gamma + sd.n) * p.V * (PT == SV_BF16 ? 2 : 4)
                       : nullptr;
    return sd;
}

// Draw stage, first kernel: the chunk sums of row n, one block per (sequence,
// chunk).  They are consumed by the next kernel, so plain stores suffice.
template <int DT, int PT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_draw_sums(const DrawParams p)
{
    const int b = (int)(blockIdx.x / (unsigned)p.nch2);
    const int c = (int)(blockIdx.x % (unsigned)p.nch2);
    __shared__ double sm_d[kWaves];
    const SeqDraw sd = seq_draw<DT, PT>(p, b);
    if (sd.invalid_seen) return;
    double E = 0.0, EA = 0.0, QA = 0.0;
    const int v0 = c * kChunk2;
    // S_row (row stage) only decides which elements lie in the residual
    // support; the normaliser itself is re-summed in fp64 here.
    if (v0 + kChunk2 <= p.V)
        draw_chunk_sums<DT, PT, VEC, true>(p, sd.zrow, sd.qrow, sd.resid, v0, sd.nMcd, sd.S_row, E, EA, QA);
    else
        draw_chunk_sums<DT, PT, VEC, false>(p, sd.zrow, sd.qrow, sd.resid, v0, sd.nMcd, sd.S_row, E, EA, QA);
    E = block_sum(E, sm_d);
    EA = block_sum(EA, sm_d);
    QA = block_sum(QA, sm_d);
    if (threadIdx.x == 0) {
        DrawPart* slot = p.part2 + (size_t)b * p.nch2 + c;
        slot->E = E;
        slot->EA = EA;
        slot->QA = QA;
    }
}

// Draw stage, second kernel: one block per sequence turns the chunk sums into
// the exact normaliser and residual mass, finds the chunk that holds the
// inverse-CDF target, scans it for the token and writes the outputs.  (A
// separate launch spreads these blocks evenly over the XCDs; run by whichever
// block of a sequence finished last, they piled up on one XCD.)
template <int DT, int PT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_draw_finish(const DrawParams p)
{
    const int b = blockIdx.x;
    const int G1 = p.gamma + 1;
    __shared__ double sm_d[kWaves];
    __shared__ int sm_i[kWaves];
    __shared__ double sm_pre;
    const SeqDraw sd = seq_draw<DT, PT>(p, b);
    const int n = sd.n;
    const bool resid = sd.resid;
    const bool invalid_seen = sd.invalid_seen;
    const void* zrow = sd.zrow;
    const void* qrow = sd.qrow;
    const double nMcd = sd.nMcd;

    // One round trip brings everything the finish needs: the chunk sums
    // (slot j cached by thread j), the uniform of the draw, and the draft
    // tokens and row statistics of the outputs.
    const int tid = (int)threadIdx.x;
    const PosInfo pi = load_pos_info(p, b);
    const double ug = (double)p.uniforms[(int64_t)b * G1 + p.gamma];
    const DrawPart* slots = p.part2 + (size_t)b * p.nch2;
    double cE = 0.0, cEA = 0.0, cQA = 0.0;
    if (tid < p.nch2) {
        cE = slots[tid].E;
        cEA = slots[tid].EA;
        cQA = slots[tid].QA;
    }
    auto slot3 = [&](int j, double& E, double& EA, double& QA) {
        if (j == tid) { E = cE; EA = cEA; QA = cQA; return; }
        E = slots[j].E; EA = slots[j].EA; QA = slots[j].QA;
    };

    const bool bad_token = tokens_invalid(p, pi, sm_i);  // called by every thread (barriers)
    const bool invalid = invalid_seen || bad_token;
    if (invalid) {
        clear_draw_partials(p, b);
        finish_sequence(p, b, n, -1, true, NAN, true, pi);
        return;
    }

    // exact normaliser of row n and the residual mass, from the chunk sums
    double S = 0.0;
    for (int j = tid; j < p.nch2; j += kThreads) {
        double E, EA, QA;
        slot3(j, E, EA, QA);
        S += E;
    }
    S = block_sum(S, sm_d);
    double Z = 0.0;
    if (resid) {
        for (int j = tid; j < p.nch2; j += kThreads) {
            double E, EA, QA;
            slot3(j, E, EA, QA);
            Z += fmax(0.0, EA / S - QA);
        }
        Z = block_sum(Z, sm_d);
    }
    // [FI] Phase 4: residual norm(max(0, p_n - q_n)) after a rejection, with
    // [ST]'s fallback to p_n; the bonus row p_gamma after full acceptance.
    const bool use_resid = resid && Z > kResidEps;
    const double total = use_resid ? Z : S;
    const double invS = 1.0 / S;  // p_v = e_v * invS (within an ulp of e_v / S)
    const double target = ug * total;
    auto chunk_weight = [&](int j) {
        double E, EA, QA;
        slot3(j, E, EA, QA);
        return use_resid ? fmax(0.0, EA / S - QA) : E;
    };

    // the first chunk whose running weight sum exceeds the target (block scan
    // over the chunk weights, kThreads chunks per round)
    int jc = -1;
    double carry = 0.0;
    for (int j0 = 0; j0 < p.nch2 && jc < 0; j0 += kThreads) {
        const int j = j0 + tid;
        const double w = j < p.nch2 ? chunk_weight(j) : 0.0;
        double tot;
        const double excl = block_exclusive_scan(w, sm_d, &tot);
        const bool hit = j < p.nch2 && w > 0.0 && carry + excl + w > target;
        const int first = block_min_i(hit ? j : INT_MAX, sm_i);
        if (first != INT_MAX) {
            if (j == first) sm_pre = carry + excl;
            __syncthreads();
            jc = first;
            carry = sm_pre;
            __syncthreads();
        } else {
            carry += tot;
        }
    }
    double rem = target - carry;  // target relative to the start of chunk jc

    // scan chunk jc (and, only if rounding pushed the crossing out of it, the
    // chunks after it) in index order: group g of thread t holds the 8
    // elements from jc * kChunk2 + (g * kThreads + t) * 8, so the groups are
    // visited g-major and, within a group, by thread.  The chunk's loads are
    // all issued before the first group is scanned.
    int tok = -1;
    while (jc >= 0 && jc < p.nch2 && tok < 0) {
        ChunkBuf<DT, PT, VEC> cb;
        cb.load(p, zrow, qrow, use_resid, jc * kChunk2);
#pragma unroll
        for (int g = 0; g < kEpt2 / 8; ++g) {
            if (tok < 0) {  // uniform
                const int idx = jc * kChunk2 + (g * kThreads + tid) * 8;
                double w[8];
                double local = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    w[e] = idx + e < p.V ? draw_weight(p, use_resid, cb.z(g, e), use_resid ? cb.q(g, e) : 0.0f, nMcd, invS)
                                         : 0.0;
                    local += w[e];
                }
                double gtot;
                const double excl = block_exclusive_scan(local, sm_d, &gtot);
                int cand = INT_MAX;
                if (excl + local > rem) {
                    double cum = excl;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        cum += w[e];
                        if (cand == INT_MAX && w[e] > 0.0 && cum > rem) cand = idx + e;
                    }
                }
                cand = block_min_i(cand, sm_i);
                if (cand != INT_MAX) tok = cand;
                rem -= gtot;
            }
        }
        ++jc;
    }
    if (tok < 0) {
        // u * total at or past the end (only by rounding, u < 1): the largest
        // index with positive weight, in the last chunk whose weight is > 0
        int jl = -1;
        for (int j = tid; j < p.nch2; j += kThreads)
            if (chunk_weight(j) > 0.0) jl = max(jl, j);
        jl = block_max_i(jl, sm_i);
        int lastv = -1;
        if (jl >= 0) {
            ChunkBuf<DT, PT, VEC> cb;
            cb.load(p, zrow, qrow, use_resid, jl * kChunk2);
#pragma unroll
            for (int g = 0; g < kEpt2 / 8; ++g) {
                const int idx = jl * kChunk2 + (g * kThreads + tid) * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (idx + e < p.V &&
                        draw_weight(p, use_resid, cb.z(g, e), use_resid ? cb.q(g, e) : 0.0f, nMcd, invS) > 0.0)
                        lastv = max(lastv, idx + e);
            }
        }
        tok = block_max_i(lastv, sm_i);
    }
    // every read of this sequence's chunk slots ended before a barrier above
    clear_draw_partials(p, b);
    finish_sequence(p, b, n, tok, false, Z, true, pi);
}

__global__ __launch_bounds__(kThreads) void k_draw_greedy(const DrawParams p)
{
    // one block per sequence: n is the first rejected position, the token the
    // argmax of row n ([FI] "Standardized Sampling", argmax case)
    const int b = blockIdx.x;
    __shared__ int sm_i[kWaves];
    __shared__ int sm_t;
    const uint64_t m = p.mask[b];
    const uint64_t rej = m & ((1ull << p.gamma) - 1ull);
    const int n = rej ? __builtin_ctzll(rej) : p.gamma;
    const PosInfo pi = load_pos_info(p, b);
    if ((int)threadIdx.x == n) sm_t = pi.st.amax;
    // every thread has read the mask before the barriers in tokens_invalid,
    // and the mask is cleared only after them (finish_sequence)
    const bool bad_token = tokens_invalid(p, pi, sm_i);
    const bool invalid = (m & kInvalidBit) != 0 || bad_token;
    finish_sequence(p, b, n, invalid ? -1 : sm_t, invalid, NAN, false, pi);
}

__global__ void k_fill_zero(uint4* p, size_t n16, unsigned char* tail, size_t ntail)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
    if (i < ntail) tail[i] = 0;
}

// ---------------------------------------------------------------- host dispatch

template <int DT>
void launch_rows(bool greedy, bool vec, int grid, const RowParams& rp, hipStream_t s)
{
    if (greedy) {
        if (vec) hipLaunchKernelGGL((k_rows_greedy<DT, true>), dim3(grid), dim3(kThreads), 0, s, rp);
        else hipLaunchKernelGGL((k_rows_greedy<DT, false>), dim3(grid), dim3(kThreads), 0, s, rp);
    } else {
        if (vec) hipLaunchKernelGGL((k_rows_sample<DT, true>), dim3(grid), dim3(kThreads), 0, s, rp);
        else hipLaunchKernelGGL((k_rows_sample<DT, false>), dim3(grid), dim3(kThreads), 0, s, rp);
    }
}

template <int DT, int PT>
void launch_draw_sample_t(bool vec, int grid_sums, int grid_finish, const DrawParams& dp, hipStream_t s)
{
    if (vec) {
        hipLaunchKernelGGL((k_draw_sums<DT, PT, true>), dim3(grid_sums), dim3(kThreads), 0, s, dp);
        hipLaunchKernelGGL((k_draw_finish<DT, PT, true>), dim3(grid_finish), dim3(kThreads), 0, s, dp);
    } else {
        hipLaunchKernelGGL((k_draw_sums<DT, PT, false>), dim3(grid_sums), dim3(kThreads), 0, s, dp);
        hipLaunchKernelGGL((k_draw_finish<DT, PT, false>), dim3(grid_finish), dim3(kThreads), 0, s, dp);
    }
}

void launch_draw_sample(int dt, int pt, bool vec, int grid_sums, int grid_finish, const DrawParams& dp,
                        hipStream_t s)
{
    if (dt == SV_FP32 && pt == SV_FP32) launch_draw_sample_t<SV_FP32, SV_FP32>(vec, grid_sums, grid_finish, dp, s);
    if (dt == SV_FP32 && pt == SV_BF16) launch_draw_sample_t<SV_FP32, SV_BF16>(vec, grid_sums, grid_finish, dp, s);
    if (dt == SV_BF16 && pt == SV_FP32) launch_draw_sample_t<SV_BF16, SV_FP32>(vec, grid_sums, grid_finish, dp, s);
    if (dt == SV_BF16 && pt == SV_BF16) launch_draw_sample_t<SV_BF16, SV_BF16>(vec, grid_sums, grid_finish, dp, s);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

size_t sv_workspace_bytes(int batch, int gamma, int vocab)
{
    if (batch < 1 || gamma < 1 || gamma > SV_MAX_GAMMA || vocab < 1) return 0;
    return make_layout(batch, gamma, vocab).total;
}

int sv_workspace_init(void* workspace, size_t bytes, void* stream)
{
    if (!workspace) return SV_ERR_NULL_POINTER;
    if (!aligned(workspace, 256)) return SV_ERR_ALIGNMENT;
    if (bytes == 0) return SV_OK;
    const size_t n16 = bytes / 16, ntail = bytes % 16;
    const size_t threads = n16 > ntail ? n16 : ntail;
    const size_t blocks = (threads + 255) / 256;
    if (blocks > (size_t)INT_MAX) return SV_ERR_TOO_LARGE;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<uint4*>(workspace), n16,
                       static_cast<unsigned char*>(workspace) + n16 * 16, ntail);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

int spec_verify(int batch, int gamma, int vocab,
                const void* target_logits, int logits_dtype,
                const void* draft_probs, int probs_dtype,
                const int32_t* draft_tokens, const float* uniforms,
                float temperature, int mode,
                int32_t* n_accepted, int32_t* out_tokens,
                void* workspace, size_t workspace_bytes,
                const sv_extras_t* extras, void* stream)
{
    // ---- argument validation (no HIP call before this block passes)
    if (mode != SV_SAMPLE && mode != SV_GREEDY) return SV_ERR_MODE;
    if (batch < 1) return SV_ERR_BATCH;
    if (gamma < 1 || gamma > SV_MAX_GAMMA) return SV_ERR_GAMMA;
    if (vocab < 1) return SV_ERR_VOCAB;
    if (logits_dtype != SV_FP32 && logits_dtype != SV_BF16) return SV_ERR_DTYPE;
    const bool greedy = mode == SV_GREEDY;
    if (!target_logits || !draft_tokens || !n_accepted || !out_tokens) return SV_ERR_NULL_POINTER;
    if (!greedy) {
        if (!draft_probs || !uniforms) return SV_ERR_NULL_POINTER;
        if (probs_dtype != SV_FP32 && probs_dtype != SV_BF16) return SV_ERR_DTYPE;
        if (!(temperature > 0.0f) || !std::isfinite(temperature)) return SV_ERR_TEMPERATURE;
    }
    const size_t lsz = logits_dtype == SV_BF16 ? 2 : 4;
    const size_t psz = probs_dtype == SV_BF16 ? 2 : 4;
    if (!aligned(target_logits, lsz) || !aligned(draft_tokens, 4) || !aligned(n_accepted, 4) ||
        !aligned(out_tokens, 4))
        return SV_ERR_ALIGNMENT;
    if (!greedy && (!aligned(draft_probs, psz) || !aligned(uniforms, 4))) return SV_ERR_ALIGNMENT;
    const Layout L = make_layout(batch, gamma, vocab);
    if (!workspace || workspace_bytes < L.total) return SV_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SV_ERR_ALIGNMENT;

    const int G1 = gamma + 1;
    const int chunk1 = logits_dtype == SV_BF16 ? kChunkBf16 : kChunkFp32;
    const int nch1 = (vocab + chunk1 - 1) / chunk1;
    const long long grid1 = (long long)G1 * batch * nch1;
    if (nch1 > 0xffff || grid1 > INT_MAX) return SV_ERR_TOO_LARGE;
    const bool vec = aligned(target_logits, 16) && ((size_t)vocab * lsz) % 16 == 0;

    const int nch2 = (vocab + kChunk2 - 1) / kChunk2;
    // draw-stage vector loads need 16-byte aligned rows in both tensors
    const bool vec2 = vocab % 8 == 0 && aligned(target_logits, 16) && (greedy || aligned(draft_probs, 16));
    const long long grid2 = greedy ? (long long)batch : (long long)batch * nch2;
    if (grid2 > INT_MAX) return SV_ERR_TOO_LARGE;

    char* ws = static_cast<char*>(workspace);
    hipStream_t s = (hipStream_t)stream;

    // log2(e)/T as c_hi + c_lo with c_hi <= log2(e)/T, so c_lo > 0 and
    // -inf logits stay -inf through both fused multiply-adds
    const double cd = greedy ? 0.0 : kLog2e / (double)temperature;
    float c_hi = (float)cd;
    if ((double)c_hi >= cd) c_hi = std::nextafter(c_hi, 0.0f);
    const float c_lo = (float)(cd - (double)c_hi);

    RowParams rp;
    rp.logits = target_logits;
    rp.probs = draft_probs;
    rp.tokens = draft_tokens;
    rp.uniforms = uniforms;
    rp.mask = reinterpret_cast<uint64_t*>(ws + L.mask_off);
    rp.cnt1 = reinterpret_cast<uint64_t*>(ws + L.cnt1_off);
    rp.part1 = reinterpret_cast<uint64_t*>(ws + L.part1_off);
    rp.stats = reinterpret_cast<RowStat*>(ws + L.stats_off);
    rp.B = batch;
    rp.gamma = gamma;
    rp.V = vocab;
    rp.nch = nch1;
    rp.probs_dtype = probs_dtype;
    rp.zero = 0u;
    rp.c_hi = c_hi;
    rp.c_lo = c_lo;
    rp.cd = cd;
    rp.ex = kExp2Coef;

    DrawParams dp;
    dp.logits = target_logits;
    dp.probs = draft_probs;
    dp.tokens = draft_tokens;
    dp.uniforms = uniforms;
    dp.mask = rp.mask;
    dp.cnt1 = rp.cnt1;
    dp.part1 = rp.part1;
    dp.nch1 = nch1;
    dp.stats = rp.stats;
    dp.part2 = reinterpret_cast<DrawPart*>(ws + L.part2_off);
    dp.n_out = n_accepted;
    dp.tok_out = out_tokens;
    dp.aux_p = extras ? extras->p_tok : nullptr;
    dp.aux_q = extras ? extras->q_tok : nullptr;
    dp.aux_resid = extras ? extras->resid_mass : nullptr;
    dp.aux_rmax = extras ? extras->row_max : nullptr;
    dp.aux_rsum = extras ? extras->row_sum : nullptr;
    dp.B = batch;
    dp.gamma = gamma;
    dp.V = vocab;
    dp.nch2 = nch2;
    dp.zero = 0u;
    dp.cd = cd;
    dp.ex = kExp2Coef;

    if (extras && extras->ev_begin && hipEventRecord((hipEvent_t)extras->ev_begin, s) != hipSuccess)
        return SV_ERR_LAUNCH;
    if (logits_dtype == SV_BF16) launch_rows<SV_BF16>(greedy, vec, (int)grid1, rp, s);
    else launch_rows<SV_FP32>(greedy, vec, (int)grid1, rp, s);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    if (extras && extras->ev_mid && hipEventRecord((hipEvent_t)extras->ev_mid, s) != hipSuccess)
        return SV_ERR_LAUNCH;
    if (greedy) hipLaunchKernelGGL(k_draw_greedy, dim3((unsigned)grid2), dim3(kThreads), 0, s, dp);
    else launch_draw_sample(logits_dtype, probs_dtype, vec2, (int)grid2, batch, dp, s);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    if (extras && extras->ev_end && hipEventRecord((hipEvent_t)extras->ev_end, s) != hipSuccess)
        return SV_ERR_LAUNCH;
    return SV_OK;
}

const char* sv_status_string(int status)
{
    switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL_POINTER: return "a required pointer is NULL";
    case SV_ERR_BATCH: return "batch must be >= 1";
    case SV_ERR_GAMMA: return "gamma must be in [1, SV_MAX_GAMMA]";
    case SV_ERR_VOCAB: return "vocab must be >= 1";
    case SV_ERR_TEMPERATURE: return "temperature must be finite and > 0 in sample mode";
    case SV_ERR_DTYPE: return "dtype must be SV_FP32 or SV_BF16";
    case SV_ERR_MODE: return "mode must be SV_SAMPLE or SV_GREEDY";
    case SV_ERR_WORKSPACE: return "workspace is NULL or smaller than sv_workspace_bytes()";
    case SV_ERR_ALIGNMENT: return "a pointer is misaligned for its element type, or the workspace is not 256-byte aligned";
    case SV_ERR_TOO_LARGE: return "problem exceeds the launch-grid limits";
    case SV_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    default: return "unknown status";
    }
}

}  // extern "C"
