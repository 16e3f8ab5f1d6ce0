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
// Sample mode is two launches on the caller's stream:
//
//   1. k_main_sample.  The grid enumerates (position k, sequence b, chunk c)
//      with k slowest.  A workgroup streams one chunk of target row (b, k)
//      with 128-bit loads and reduces it to a partial (max, sum of exp); the
//      last workgroup of a row (arrival counter) merges the row's partials,
//      takes the acceptance decision for position k and publishes the row's
//      statistics.  Rows past the first rejection are never needed ([FI]
//      Phase 3: the walk stops at the first rejection), so a workgroup that
//      finds an earlier position of its sequence rejected skips its chunk;
//      with position-major launch order most unneeded rows are never read.
//      The decider that completes a sequence's decisions appends it, with
//      its n, to a ready list.  After every row workgroup the grid holds the
//      draw helpers: for each rank of the ready list one per draw chunk (one
//      per sub-chunk in the smallest batches); a helper waits (bounded) for
//      its rank's sequence and computes the fp64 sums of its part of row n
//      (the residual max(0, p_n - q_n), or p_gamma when n = gamma), so the
//      draws of the sequences resolved first overlap the rows of the others.
//      For batches whose positions hold few row workgroups the launch takes
//      dynamic LDS that caps its resident workgroups per CU, so that later
//      positions do not stream rows ahead of the decisions that skip them.
//
//   2. k_finish_sample, one workgroup per sequence: it computes any draw
//      chunk no helper did, turns the sums into the inverse-CDF draw (its
//      four waves scanning the chosen sub-chunk's four groups side by side),
//      writes the outputs and clears the sequence's workspace.  (Calls that ask for
//      the acceptance telemetry stream every row and sweep the rows between
//      the launches; their last launch is k_rest_sample.)
//
// Greedy mode is k_rows_greedy (same grid; chunk argmax; half-size chunks of
// bf16 rows for small batches) and k_draw_greedy.
//
// Numerics.  The row stage uses fp32 exp2 with a two-term log2(e)/T and a
// per-chunk correction of the rounded shift, and accumulates in fp64; the
// acceptance threshold is formed in fp64.  The draw works entirely in fp64
// (e_v, normaliser, residual, prefix sums), so its token boundaries agree
// with an fp64 evaluation to rounding level.
//
// Cross-workgroup data within a launch (row statistics, and the draw sums
// of k_rest_sample) are written with device-scope atomic exchanges whose
// returned values feed the operand of the atomic that announces them (a
// decision bit, a completion count), so they are complete device-wide
// before anyone can learn of them; readers use device-scope atomic loads.
// Row partials go out with device-scope stores whose words are never zero,
// and the row's last workgroup polls each slot until both have landed.
//
// Workspace: per-sequence control words and per-row arrival counters, then
// scratch for partials, row statistics and draw sums.  It must be all zero
// before a call; the last user of each sequence's part clears it, so a
// finished call leaves all of it zero again, whatever shape the next call
// has.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint64_t kInvalidBit = 1ull << 63;
// A ready-list entry: (b + 1) | n << kReadyNShift, so that whoever reads a
// sequence's entry learns its n in the same load (sample mode limits B to
// kMaxListed).
constexpr int kReadyNShift = 26;
constexpr uint32_t kReadySeqMask = (1u << kReadyNShift) - 1u;
constexpr int kMaxListed = (int)kReadySeqMask - 1;
// SeqCtl::pad[0], bit k: the merge of row k ran out of its bounded wait for a
// partial (the sequence's outputs are withheld if k is on its walk, k <= n)
constexpr double kResidEps = 1e-15;  // [ST] correction_distribution
constexpr double kLog2e = 1.4426950408889634073599246810018921;

// Elements per thread of one row-stage chunk (a chunk is 32 KiB of input).
constexpr int kEptBf16 = 64;
constexpr int kEptFp32 = 32;
constexpr int kChunkBf16 = kEptBf16 * kThreads;  // 16384 elements
constexpr int kChunkFp32 = kEptFp32 * kThreads;  // 8192 elements

// Draw geometry.  A group is 512 consecutive elements of row n, 8 per lane
// of one wave; a wave task is 4 consecutive groups, a sub-chunk of 2048
// elements whose sums the wave publishes (loaded in passes of 2 groups in
// the first launch, which keeps the fused row kernel at 8 waves per SIMD),
// and a draw chunk (one claim) is the 4 waves of a workgroup: 8192 elements.
constexpr int kSub = 512;                           // elements of a group
constexpr int kSubPerWave = 4;                      // groups of a wave task (one sub-chunk)
constexpr int kSubPerPass = 2;  // first launch (the helpers share SIMDs with the row stage)
// Up to this many sub-chunks in a batch, the first launch's draw helpers take
// one sub-chunk each (a group per wave) rather than a draw chunk each: four
// times the helpers, each a quarter as long, for batches whose helpers all fit
// on the chip at once (~one round of resident workgroups at the cap of 3 per
// CU), where the draws sit on the call's critical path.  Above it the extra
// helpers' fixed costs (the ready-list poll, the row statistics) outweigh the
// shorter draws.
constexpr long long kFineHelpers = 1024;
// Greedy calls on bf16 rows take kChunkFp32-entry row chunks when a position has
// at most this many kChunkBf16-entry ones: with few rows the decisions, not the
// streaming, set the pace, and shorter blocks reach them sooner (the cap on
// resident row blocks then comes out at 8: none).
constexpr long long kHalfChunkBlocks = 1024;
constexpr int kSubPerChunk = kSubPerWave * kWaves;  // 16 groups in a draw chunk
constexpr int kChunk2 = kSub * kSubPerChunk;        // 8192
constexpr int kSubW = kSub * kSubPerWave;           // 2048 elements of a sub-chunk
constexpr int kRPL = 2;                             // sub-chunk sums per lane per finish round
constexpr int kRound = 64 * kRPL;                   // sub-chunk sums per finish round
constexpr int kChunkB = 8192;                       // telemetry sweep: row elements per workgroup
constexpr int kGroupsB = kChunkB / (8 * kThreads);  // groups of 8 per thread
static_assert(kChunkB == kChunk2, "a telemetry workgroup covers exactly one draw chunk");
static_assert(kChunk2 == kSubW * kWaves, "a draw chunk is one sub-chunk per wave");
static_assert(kSubPerWave == kWaves, "the last launch scans a sub-chunk's groups one per wave");
// Bound of a draw helper's wait for its sequence to be resolved (polls ~1 us
// apart under load; the row stage of a call takes ~100 us at most).
constexpr int kHelpPolls = 1 << 14;


// Per-row statistics written by the row stage.
struct RowStat {
    float m;       // row max of the raw logits
    int32_t amax;  // greedy: first index attaining m
    double S;      // sum_v exp((z_v - m)/T)
    double P;      // p_k(x_k)
    double Q;      // q_k(x_k)
};
static_assert(sizeof(RowStat) == 32, "RowStat layout");

// Draw sums of one sub-chunk of row n.
struct SubSum {
    double E;   // sum of e_v = exp((z_v - m)/T)
    double EA;  // sum of e_v over A = {v : e_v > q_v S_row} (residual support)
    double QA;  // sum of q_v over A
    double done;  // nonzero once a first-launch draw helper has written the three sums
};
static_assert(sizeof(SubSum) == 32, "SubSum layout");

// Per-sequence control words.
struct SeqCtl {
    uint64_t mask;    // bit k: position k rejected; kInvalidBit: a bad draft token
    uint64_t dec;     // bit k: position k decided (a rejection also sets every
                      // later bit); bit gamma: row gamma's statistics out
    uint64_t claim;   // telemetry calls: draw chunks claimed before the last launch,
                      // in order: chunks 0 .. claim-1 (claims past nch2 take nothing)
    uint64_t cnt2;    // draw wave tasks finished in the second launch
    uint64_t retire;  // low word: users done in the second launch; high word:
                      // the sequence's rank in the ready list
    uint64_t pad[3];
};
static_assert(sizeof(SeqCtl) == 64, "SeqCtl layout");

struct Layout {
    size_t ctl_off, cnt1_off, ready_off, rcnt_off, control_bytes;
    size_t part1_off, stats_off, sub_off, bpart_off, total;
    int nch1_max, nch2, nsub, nchb;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout make_layout(int B, int gamma, int V)
{
    Layout L;
    const size_t rows = (size_t)B * (size_t)(gamma + 1);
    L.nch1_max = (V + kChunkFp32 - 1) / kChunkFp32;
    L.nch2 = (V + kChunk2 - 1) / kChunk2;
    L.nsub = L.nch2 * kWaves;  // sub-chunks of kSubW elements
    L.nchb = (V + kChunkB - 1) / kChunkB;
    size_t off = 0;
    L.ctl_off = off;   off = align256(off + sizeof(SeqCtl) * (size_t)B);
    L.cnt1_off = off;  off = align256(off + sizeof(uint64_t) * rows);
    L.ready_off = off; off = align256(off + sizeof(int32_t) * (size_t)B);
    L.rcnt_off = off;  off = align256(off + sizeof(uint32_t));
    L.control_bytes = off;
    L.part1_off = off; off = align256(off + 2 * sizeof(uint64_t) * rows * (size_t)L.nch1_max);
    L.stats_off = off; off = align256(off + sizeof(RowStat) * rows);
    L.sub_off = off;   off = align256(off + sizeof(SubSum) * (size_t)B * (size_t)L.nsub);
    L.bpart_off = off; off = align256(off + sizeof(double) * (size_t)B * (size_t)gamma * (size_t)L.nchb);
    L.total = off;
    return L;
}

// ------------------------------------------------------------------ device helpers

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p)
{
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_agent_d(const double* p)
{
    return __longlong_as_double((long long)ld_agent(reinterpret_cast<const uint64_t*>(p)));
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent32(const uint32_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t xchg_agent(uint64_t* p, uint64_t v)
{
    return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t or_agent(uint64_t* p, uint64_t v)
{
    return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t add_agent64(uint64_t* p, uint64_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fold64(uint64_t v) { return (uint32_t)(v ^ (v >> 32)); }
__device__ __forceinline__ uint64_t dbits(double d) { return (uint64_t)__double_as_longlong(d); }

// Publishes words for the last reader: each goes out with a device-scope
// atomic exchange, and the caller makes the exchanged-out old values an
// operand of the atomic that announces the data, so every exchange has
// completed device-wide before that announcement can be observed.  (A
// release/acquire pair at agent scope orders the same thing but writes back
// the whole L2 on every workgroup, about ten times the cost of the streaming
// work itself.)  `zero` is a kernel argument that is always 0 and opaque to
// the compiler; the result is always 0.
template <int N>
__device__ __forceinline__ uint32_t publish(uint64_t* slot, const uint64_t (&w)[N], uint32_t zero)
{
    uint64_t dep = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) dep ^= xchg_agent(slot + i, w[i]);
    return fold64(dep) & zero;
}

__device__ __forceinline__ uint64_t stat_word0(float m, int32_t amax)
{
    return (uint64_t)__float_as_uint(m) | ((uint64_t)(uint32_t)amax << 32);
}
__device__ __forceinline__ RowStat ld_stat(const RowStat* s)
{
    const uint64_t* w = reinterpret_cast<const uint64_t*>(s);
    const uint64_t w0 = ld_agent(w), w1 = ld_agent(w + 1), w2 = ld_agent(w + 2), w3 = ld_agent(w + 3);
    RowStat r;
    r.m = __uint_as_float((uint32_t)w0);
    r.amax = (int32_t)(uint32_t)(w0 >> 32);
    r.S = __longlong_as_double((long long)w1);
    r.P = __longlong_as_double((long long)w2);
    r.Q = __longlong_as_double((long long)w3);
    return r;
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
__device__ __forceinline__ uint32_t wave_xor(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v ^= (uint32_t)__shfl_xor((int)v, o, 64);
    return v;
}
// Inclusive prefix sum over the 64 lanes of a wave (lane order).
__device__ __forceinline__ double wave_incl_scan(double v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}
__device__ __forceinline__ int first_lane(uint64_t ballot) { return ballot ? __builtin_ctzll(ballot) : -1; }

// The same sum and scan with DPP lane moves instead of LDS permutes, for
// the single-wave, latency-bound draw finish (each step is a few cycles
// instead of a round trip through the LDS crossbar).  The double moves as
// two 32-bit halves; lanes without a source read 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ double dpp_d(double v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xf, false);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_sum_dpp(double v)
{
    v += dpp_d<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_d<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_d<0x141>(v);  // row_half_mirror
    v += dpp_d<0x140>(v);  // row_mirror: every lane holds its 16-lane row's sum
    const double r0 = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 0), __builtin_amdgcn_readlane(__double2loint(v), 0));
    const double r1 = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 16), __builtin_amdgcn_readlane(__double2loint(v), 16));
    const double r2 = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 32), __builtin_amdgcn_readlane(__double2loint(v), 32));
    const double r3 = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 48), __builtin_amdgcn_readlane(__double2loint(v), 48));
    return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ double wave_incl_scan_dpp(double v)
{
    v += dpp_d<0x111>(v);        // row_shr:1
    v += dpp_d<0x112>(v);        // row_shr:2
    v += dpp_d<0x114>(v);        // row_shr:4
    v += dpp_d<0x118>(v);        // row_shr:8: scans within each row
    v += dpp_d<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_d<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
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
    wave_amax(v, i);
    if ((threadIdx.x & 63) == 0) { smf[threadIdx.x >> 6] = v; smi[threadIdx.x >> 6] = i; }
    __syncthreads();
    v = smf[0]; i = smi[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) amax_merge(v, i, smf[w], smi[w]);
    __syncthreads();
}

// 2^a in double for a <= 0, relative error below 5.6e-11 (the draw's token
// boundaries are judged in a 1e-9 relative window; a residual boundary,
// which subtracts l q_v from each p_v, carries the error as an absolute one,
// so its relative error grows as the target's mass on the residual's support
// over the residual mass): a = k + f with k the nearest
// integer (rounded by adding 1.5 * 2^52, which leaves k in the low word) and
// |f| <= 1/2; 2^f by the degree-7 polynomial interpolating it at the 8
// Chebyshev nodes of [-1/2, 1/2] (seven fused multiply-adds, the constant
// term included); 2^k applied with ldexp, which rounds to a subnormal or to
// 0 below the normal range.  a is clamped at
// -1100 first, so -inf gives exactly 0.  The coefficients travel as kernel
// arguments: uniform values stay in scalar registers, which fp64 FMAs read
// directly (as literals they would be rebuilt in vector registers for every
// element); the clamp and the rounding constant have 32-bit literal forms.
struct Exp2Coef {
    double c[8];  // c[0] multiplies f^7, c[6] multiplies f, c[7] is the constant term
};
constexpr Exp2Coef kExp2Coef = {{1.5303700711009567e-05, 0.00015469729214112252, 0.0013333478473687005,
                                 0.009618025613318053, 0.055504109063258644, 0.24022651213498092,
                                 0.6931471805568324, 0.9999999999595618}};

__device__ __forceinline__ double exp2_f64(double a, const Exp2Coef& k)
{
    constexpr double kMagic = 6755399441055744.0;  // 1.5 * 2^52
    a = __builtin_fmax(a, -1100.0);
    const double t = a + kMagic;
    const double f = a - (t - kMagic);
    const int n = __double2loint(t);
    double p = k.c[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) p = fma(f, p, k.c[i]);
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
    // Signed 16-bit maximum of the raw bf16 patterns (bf16 vector path): it
    // is the float maximum whenever it is >= 0 (a positive pattern exceeds
    // every negative one, and positive patterns order like their values).
    __device__ __forceinline__ int max_bits16() const
    {
        typedef short s2 __attribute__((ext_vector_type(2)));
        s2 acc = __builtin_bit_cast(s2, raw[0].x);
#pragma unroll
        for (int j = 0; j < EPT / W; ++j) {
            if (j > 0) acc = __builtin_elementwise_max(acc, __builtin_bit_cast(s2, raw[j].x));
            acc = __builtin_elementwise_max(acc, __builtin_bit_cast(s2, raw[j].y));
            acc = __builtin_elementwise_max(acc, __builtin_bit_cast(s2, raw[j].z));
            acc = __builtin_elementwise_max(acc, __builtin_bit_cast(s2, raw[j].w));
        }
        return max((int)acc.x, (int)acc.y);
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

// 8 consecutive elements as raw 128-bit words (one for bf16, two for fp32).
struct Raw8 {
    uint4 a, b;
};
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

// The 8 elements idx .. idx+7 of a row.  Vector path (idx a multiple of 8,
// 16-byte aligned row): 128-bit loads, the address clamped to the row when
// the group ends past V (the caller ignores elements >= V).  Scalar path:
// element loads, indices clamped to the row.
template <int DT, bool VEC2>
__device__ __forceinline__ Raw8 load_group(const void* rowp, int idx, int V)
{
    constexpr size_t ES = DT == SV_BF16 ? 2 : 4;
    Raw8 r;
    if constexpr (VEC2) {
        const int ci = min(idx, V - 8);
        const char* ptr = static_cast<const char*>(rowp) + (size_t)ci * ES;
        r.a = *reinterpret_cast<const uint4*>(ptr);
        if constexpr (DT == SV_FP32) r.b = *reinterpret_cast<const uint4*>(ptr + 16);
        else r.b = make_uint4(0u, 0u, 0u, 0u);
    } else {
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = min(idx + e, V - 1);
            if constexpr (DT == SV_BF16) w[e] = static_cast<const uint16_t*>(rowp)[i];
            else w[e] = static_cast<const uint32_t*>(rowp)[i];
        }
        if constexpr (DT == SV_BF16) {
            r.a = make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16));
            r.b = make_uint4(0u, 0u, 0u, 0u);
        } else {
            r.a = make_uint4(w[0], w[1], w[2], w[3]);
            r.b = make_uint4(w[4], w[5], w[6], w[7]);
        }
    }
    return r;
}

// ------------------------------------------------------------------ parameters

struct Params {
    const void* logits;
    const void* probs;
    const int32_t* tokens;
    const float* uniforms;
    SeqCtl* ctl;
    uint64_t* cnt1;   // per row: arrivals (low 16 bits), rejection evidence (high 48)
    uint64_t* part1;  // [rows][nch1][2]
    RowStat* stats;   // [rows]
    SubSum* sub;      // [B][nsub] sums of the sub-chunks (kSubW elements) of row n
    uint32_t* ready;  // [B] the sequences, in the order their n became known (ready-list entries)
    uint32_t* ready_cnt;
    int32_t* n_out;
    int32_t* tok_out;
    double* aux_p;
    double* aux_q;
    double* aux_resid;
    double* aux_pout;  // [B] p_n(t) of the drawn token
    float* aux_rmax;
    double* aux_rsum;
    int B, gamma, V, nch1, nch2, nsub, probs_dtype;
    double* aux_beta;  // telemetry outputs (see sv_extras_t), or NULL
    double* aux_alpha;
    double* bpart;     // [B][gamma][nchb] telemetry partial sums
    int tele, nchb;    // tele: every row is streamed and the telemetry sweep runs
    uint32_t zero;     // always 0 (see publish)
    float c_hi, c_lo;  // log2(e)/T split into two fp32 terms, c_lo > 0
    double cd;         // log2(e)/T in double
    double len;        // lenience l in [0, 1] (1: the exact method)
    Exp2Coef ex;       // kExp2Coef
    int rows_grid;     // first launch: row blocks (G1 * B * nch1); the draw helpers follow
    int help_polls;    // bound of a draw helper's wait for its sequence
    int fine;          // 1: one draw helper per sub-chunk (a wave per group), else one per draw chunk
    int polls_slot;    // bound of a merge's wait for a partial slot
    int drop_slot;     // test hook: >= 0 makes chunk 0 of that position withhold its
                       // partial, so that the merge's bounded wait runs out
    uint32_t* err_count;  // optional: sequences whose merge wait ran out
};

__device__ __forceinline__ int ready_seq(uint32_t e) { return (int)(e & kReadySeqMask) - 1; }
__device__ __forceinline__ int ready_n(uint32_t e) { return (int)(e >> kReadyNShift); }

// Which part of the work a workgroup takes, from its index.  Host and
// device: the kernels decode their blocks with these, and a CPU test checks
// them against the launch geometry and the workspace layout.
struct RowBlock {
    int k, b, c;  // position, sequence, chunk of the row stage
};
__host__ __device__ __forceinline__ RowBlock row_block(uint32_t bid, int nch1, int B)
{
    const uint32_t t = bid / (uint32_t)nch1;  // k * B + b
    return RowBlock{(int)(t / (uint32_t)B), (int)(t % (uint32_t)B), (int)(bid % (uint32_t)nch1)};
}
struct DrawTask {
    int r, c2;  // rank in the ready list, draw chunk
};
__host__ __device__ __forceinline__ DrawTask helper_task(int j, int nch2)
{
    const int r = j / nch2;
    return DrawTask{r, j - r * nch2};
}
// the sub-chunk (kSubW elements, one wave task) of wave w of draw chunk c2
__host__ __device__ __forceinline__ int wave_sub(int c2, int w) { return c2 * kWaves + w; }
// fine helpers: helper j takes sub-chunk j % nsub of the (j / nsub)-th listed
// sequence, its wave w group w of that sub-chunk
__host__ __device__ __forceinline__ DrawTask fine_task(int j, int nsub)
{
    const int r = j / nsub;
    return DrawTask{r, j - r * nsub};
}
struct BetaBlock {
    int b, i, c;  // sequence, position, telemetry chunk
};
__host__ __device__ __forceinline__ BetaBlock beta_block(uint32_t bid, int nchb, int gamma)
{
    const int t = (int)(bid / (uint32_t)nchb);  // b * gamma + i
    const int b = t / gamma;
    return BetaBlock{b, t - b * gamma, (int)(bid % (uint32_t)nchb)};
}
struct RestTask {
    int r, j;  // rank in the ready list, the sequence's workgroup
};
__host__ __device__ __forceinline__ RestTask rest_task(int i, int B, int nch2)
{
    const int per = nch2 - 1 > 1 ? nch2 - 1 : 1;
    if (i < B) return RestTask{B - 1 - i, 0};
    return RestTask{B - 1 - (i - B) / per, 1 + (i - B) % per};
}

// bits 0 .. gamma (one per row of a sequence)
__device__ __forceinline__ uint64_t rows_mask(int gamma) { return (2ull << gamma) - 1ull; }
// n from a reject mask: the first rejected position, gamma if none
__device__ __forceinline__ int first_reject(uint64_t mask, int gamma)
{
    const uint64_t rej = mask & ((1ull << gamma) - 1ull);
    return rej ? __builtin_ctzll(rej) : gamma;
}

// ------------------------------------------------------------- row stage helpers

// The counter word of a row also gathers evidence of a rejection (sample
// mode): each block adds, in its high 48 bits, floor(2^30 min(2, u Q s'))
// where s' is its chunk's sum of exp((z_v - z_x)/T) (z_x the draft token's
// logit).  Every term is positive, so once the running total exceeds 2^30
// (plus a margin far above the rounding of these terms)
// u Q sum_v exp((z_v - z_x)/T) > 1, i.e. p(x) / q(x) < u: the position is
// rejected whatever the other chunks hold.  The block that sees this sets
// the reject bit at once, so later positions of the sequence stop being
// fetched sooner; the last block still takes the full decision, which is
// the same.
constexpr int kCountBits = 16;
// merge of a row's partials: slots per lane per pass, and the bound of the
// wait for a slot whose store is still in flight
constexpr int kMaxSlotsPerLane = 1;
constexpr int kSlotPolls = 1 << 20;  // default bound of a merge's wait for a partial (~28 ms)
constexpr uint64_t kSlotFlag = 1ull << 32;  // above the max's float bits in a partial's first word
constexpr uint64_t kSignBit = 1ull << 63;
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

// Run by thread 0's wave once the block's reductions are done: count this
// block in and learn whether it is the last block of the row; the last
// block resets the counter to zero.  Blocks that skip their chunk never
// count in, so a row with a skipped chunk has no last block (it is not
// needed: an earlier position was rejected); the sequence's last user
// clears such a row's counter.
__device__ __forceinline__ bool row_arrive(const Params& p, int64_t row, int b, uint64_t evidence,
                                          uint64_t early_bit, uint32_t dep)
{
    uint32_t last = 0;
    if (threadIdx.x == 0) {
        // a chunk whose own evidence settles the rejection sets the bit at
        // once, a round trip before the count's old value could
        if (early_bit && evidence > kEvidenceThreshold) or_agent(&p.ctl[b].mask, early_bit);
        const uint64_t add = 1ull + (evidence << kCountBits) + dep;
        const uint64_t old = __hip_atomic_fetch_add(&p.cnt1[row], add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = (old & kCountMask) + 1ull == (uint64_t)p.nch1 ? 1u : 0u;
        if (last) {
            __hip_atomic_store(&p.cnt1[row], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (early_bit && (old >> kCountBits) + evidence > kEvidenceThreshold) {
            or_agent(&p.ctl[b].mask, early_bit);
        }
    }
    return __builtin_amdgcn_readfirstlane(last) != 0u;
}

// ------------------------------------------------------------------ draw

// This lane's share of the sums over groups s0 .. s0+NP-1 of row n of
// sequence b, in fp64, added to E, EA, QA: E = sum e_v with
// e_v = 2^((z_v - m) log2(e)/T) (m the row max; the shift -m log2(e)/T is
// rounded once for the row, a common factor that cancels in every ratio
// used), and for a residual draw EA, QA over A = {v : e_v > q_v S_row}.
// S_row, the row stage's normaliser, only decides membership of A; the exact
// normaliser is the sum of E.
template <int DT, int PT, bool VEC2, int NP>
__device__ __forceinline__ void draw_wave_load(const Params& p, const void* zrow, const void* qrow, bool resid,
                                               int s0, Raw8 (&zr)[NP], Raw8 (&qr)[NP])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int g = 0; g < NP; ++g) zr[g] = load_group<DT, VEC2>(zrow, (s0 + g) * kSub + lane * 8, p.V);
    if (resid) {
#pragma unroll
        for (int g = 0; g < NP; ++g) qr[g] = load_group<PT, VEC2>(qrow, (s0 + g) * kSub + lane * 8, p.V);
    }
}
template <int DT, int PT, bool VEC2, bool RESID, bool FULL, int NP>
__device__ __forceinline__ void draw_wave_sums(const Params& p, const Raw8 (&zr)[NP], const Raw8 (&qr)[NP], int s0,
                                               double nMcd, double S_row, double& E, double& EA, double& QA)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int g = 0; g < NP; ++g) {
        const int idx = (s0 + g) * kSub + lane * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool ok = FULL || idx + e < p.V;
            double ev = exp2_f64(fma((double)raw8_elem<DT>(zr[g], e), p.cd, nMcd), p.ex);
            if constexpr (!FULL) ev = ok ? ev : 0.0;
            E += ev;
            if constexpr (RESID) {
                const double qd = (double)raw8_elem<PT>(qr[g], e);
                // 1.0 if v is in the residual support, else 0.0
                const double in = __hiloint2double((ok && ev > qd * S_row) ? 0x3ff00000 : 0, 0);
                EA = fma(ev, in, EA);
                QA = fma(qd, in, QA);
            }
        }
    }
}

// COUNTED (the last launch): the sums go out with device-scope exchanges
// and the wave counts itself in; returns true in the wave whose count
// reaches `target` (the sequence's wave tasks in that launch), which
// completes the sequence's draw sums.  Otherwise (the first launch's draw
// helpers, the telemetry sweep) plain stores with a done mark, which the
// last launch reads after the kernel boundary.
template <int DT, int PT, bool VEC2, bool COUNTED>
__device__ bool draw_wave(const Params& p, int b, int s0, uint64_t mask, uint64_t target)
{
    const int lane = threadIdx.x & 63;
    const int n = first_reject(mask, p.gamma);
    const bool resid = n < p.gamma;
    const int64_t row = (int64_t)b * (p.gamma + 1) + n;
    uint64_t dep = 0;
    const void* zrow = static_cast<const char*>(p.logits) + (size_t)row * p.V * (DT == SV_BF16 ? 2 : 4);
    const void* qrow = static_cast<const char*>(p.probs) +
                       (size_t)((int64_t)b * p.gamma + (resid ? n : 0)) * p.V * (PT == SV_BF16 ? 2 : 4);
    // the second launch sits on the critical path with SIMDs to spare: all of
    // a wave's groups in one load pass there
    constexpr int NP = COUNTED ? kSubPerWave : kSubPerPass;
    double E = 0.0, EA = 0.0, QA = 0.0;  // this lane's share of the sub-chunk's sums
    if (!(mask & kInvalidBit)) {
        // the first pass's elements are on their way before the row's
        // statistics are asked for
        Raw8 zr[NP], qr[NP];
        draw_wave_load<DT, PT, VEC2, NP>(p, zrow, qrow, resid, s0, zr, qr);
        const uint64_t* sw = reinterpret_cast<const uint64_t*>(p.stats + row);
        const double nMcd = -(double)__uint_as_float((uint32_t)ld_agent(sw)) * p.cd;
        // (only decides membership of A = {v : e_v > l q_v S}: scaled by the lenience)
        const double S_row = p.len * __longlong_as_double((long long)ld_agent(sw + 1));
#pragma unroll
        for (int s = s0; s < s0 + kSubPerWave; s += NP) {
            if (s > s0) draw_wave_load<DT, PT, VEC2, NP>(p, zrow, qrow, resid, s, zr, qr);
            const bool full = (s + NP) * kSub <= p.V;
            if (resid) {
                if (full) draw_wave_sums<DT, PT, VEC2, true, true, NP>(p, zr, qr, s, nMcd, S_row, E, EA, QA);
                else draw_wave_sums<DT, PT, VEC2, true, false, NP>(p, zr, qr, s, nMcd, S_row, E, EA, QA);
            } else {
                if (full) draw_wave_sums<DT, PT, VEC2, false, true, NP>(p, zr, qr, s, nMcd, S_row, E, EA, QA);
                else draw_wave_sums<DT, PT, VEC2, false, false, NP>(p, zr, qr, s, nMcd, S_row, E, EA, QA);
            }
        }
    }
    E = wave_sum(E);
    EA = wave_sum(EA);
    QA = wave_sum(QA);
    const int sidx = s0 / kSubPerWave;  // this wave task's sub-chunk
    if (lane == 0) {
        if constexpr (COUNTED) {
            uint64_t* slot = reinterpret_cast<uint64_t*>(p.sub + (size_t)b * p.nsub + sidx);
            dep ^= xchg_agent(slot, dbits(E)) ^ xchg_agent(slot + 1, dbits(EA)) ^ xchg_agent(slot + 2, dbits(QA));
        } else {
            p.sub[(size_t)b * p.nsub + sidx] = SubSum{E, EA, QA, 1.0};
        }
    }
    if constexpr (COUNTED) {
        const uint32_t d = wave_xor(fold64(dep)) & p.zero;
        uint32_t last = 0;
        if (lane == 0) last = __hip_atomic_fetch_add(&p.ctl[b].cnt2, 1ull + d, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) + 1ull == target ? 1u : 0u;
        return __builtin_amdgcn_readfirstlane(last) != 0u;
    }
    return false;
}

// Group grp (kSub elements) of the draw row of sequence b, n from `mask`:
// the wave's totals of E, EA, QA (see draw_wave_load), for a fine helper.
template <int DT, int PT, bool VEC2>
__device__ void draw_group(const Params& p, int b, int grp, uint64_t mask, double& E, double& EA, double& QA)
{
    const int n = first_reject(mask, p.gamma);
    const bool resid = n < p.gamma;
    const int64_t row = (int64_t)b * (p.gamma + 1) + n;
    const void* zrow = static_cast<const char*>(p.logits) + (size_t)row * p.V * (DT == SV_BF16 ? 2 : 4);
    const void* qrow = static_cast<const char*>(p.probs) +
                       (size_t)((int64_t)b * p.gamma + (resid ? n : 0)) * p.V * (PT == SV_BF16 ? 2 : 4);
    E = EA = QA = 0.0;
    if (!(mask & kInvalidBit) && grp * kSub < p.V) {
        Raw8 zr[1], qr[1];
        draw_wave_load<DT, PT, VEC2, 1>(p, zrow, qrow, resid, grp, zr, qr);
        const uint64_t* sw = reinterpret_cast<const uint64_t*>(p.stats + row);
        const double nMcd = -(double)__uint_as_float((uint32_t)ld_agent(sw)) * p.cd;
        const double S_row = p.len * __longlong_as_double((long long)ld_agent(sw + 1));
        const bool full = (grp + 1) * kSub <= p.V;
        if (resid) {
            if (full) draw_wave_sums<DT, PT, VEC2, true, true, 1>(p, zr, qr, grp, nMcd, S_row, E, EA, QA);
            else draw_wave_sums<DT, PT, VEC2, true, false, 1>(p, zr, qr, grp, nMcd, S_row, E, EA, QA);
        } else {
            if (full) draw_wave_sums<DT, PT, VEC2, false, true, 1>(p, zr, qr, grp, nMcd, S_row, E, EA, QA);
            else draw_wave_sums<DT, PT, VEC2, false, false, 1>(p, zr, qr, grp, nMcd, S_row, E, EA, QA);
        }
    }
    E = wave_sum(E);
    EA = wave_sum(EA);
    QA = wave_sum(QA);
}

// Element i of a row of logits or probabilities, as float.
template <int DT>
__device__ __forceinline__ float elem_at(const void* row, int64_t i)
{
    if constexpr (DT == SV_BF16) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(row)[i] << 16);
    else return static_cast<const float*>(row)[i];
}

// Weight of one element of row n for the inverse-CDF draw: max(0, p - l q)
// with p = e / S and l the lenience (1: the exact method), or e itself for
// the bonus / fallback draw.
__device__ __forceinline__ double draw_weight(const Params& p, bool use_resid, float z, float q, double nMcd,
                                              double invS)
{
    const double e = exp2_f64(fma((double)z, p.cd, nMcd), p.ex);
    return use_resid ? fmax(0.0, e * invS - p.len * (double)q) : e;
}

// Clears everything the call left in the workspace for sequence b.  Run by
// one wave, by the sequence's last user.  `listed`: the sequence is in the
// ready list (sample mode), at `rank`.  With `exchange` it leaves the list
// first: a second-launch workgroup that reads the control words and then
// still finds the sequence listed has read them before they were cleared,
// since every clearing store is issued only once the exchange has returned
// (its value feeds their addresses).  Without it (no other workgroup reads
// the sequence's workspace any more) the list entry is simply cleared.
__device__ void cleanup_wave(const Params& p, int b, uint32_t rank, bool listed, bool exchange = true)
{
    const int lane = threadIdx.x & 63;
    const int G1 = p.gamma + 1;
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    uint32_t d = 0;
    if (listed && lane == 0) {
        if (exchange) {
            d = __hip_atomic_exchange(&p.ready[rank], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (rank == 0) d ^= __hip_atomic_exchange(p.ready_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            p.ready[rank] = 0u;
            if (rank == 0) *p.ready_cnt = 0u;
        }
    }
    const size_t dz = __builtin_amdgcn_readfirstlane(d) & p.zero;
    if (lane < 4) reinterpret_cast<uint4*>(p.ctl + b + dz)[lane] = z4;
    for (int i = lane; i < G1; i += 64) p.cnt1[(int64_t)b * G1 + dz + i] = 0ull;
    uint4* part = reinterpret_cast<uint4*>(p.part1 + 2 * (size_t)b * G1 * p.nch1 + dz);
    for (int j = lane; j < G1 * p.nch1; j += 64) part[j] = z4;
    uint4* st = reinterpret_cast<uint4*>(p.stats + (size_t)b * G1 + dz);
    for (int j = lane; j < 2 * G1; j += 64) st[j] = z4;
    uint4* ss = reinterpret_cast<uint4*>(p.sub + (size_t)b * p.nsub + dz);
    for (int j = lane; j < 2 * p.nsub; j += 64) ss[j] = z4;
}

// Counts one user of sequence b out in the second launch (each of its
// workgroups with work there, and the draw); the last of the `users` clears
// the sequence.  Called by one wave after its reads of the sequence's
// workspace.
__device__ __forceinline__ void retire_wave(const Params& p, int b, uint32_t users)
{
    uint64_t old = 0;
    if ((threadIdx.x & 63) == 0)
        old = __hip_atomic_fetch_add(&p.ctl[b].retire, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)old);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(old >> 32));
    if (lo + 1u == users) cleanup_wave(p, b, hi, true);
}

// The draw of sequence b and its outputs, by one wave, once every
// sub-chunk sum is out ([FI] Phase 4: the residual norm(max(0, p_n - q_n)) after a
// rejection, with [ST]'s fallback to p_n; the bonus row p_gamma after full
// acceptance).  The exact normaliser S and residual mass Z come from the
// sub-chunk sums; a scan over the sub-chunk weights in index order finds the
// sub-chunk holding u * total, and a scan of its elements, a 512-element
// group at a time with every weight recomputed exactly, finds the token.
// MARKS: the sums come from the first launch's draw helpers, each with its
// done mark; if a mark is missing the wave writes nothing and returns false.
// PAR: every wave of the workgroup runs this on the same data (so all take
// the same branches and meet at the barriers), wave w scans group w of the
// sub-chunk and the groups' totals are combined through LDS in index order,
// the sequential scan's arithmetic unchanged; wave 0 writes the outputs.
template <int DT, int PT, bool VEC2, bool MARKS, bool PAR = false>
__device__ bool finish_wave(const Params& p, int b)
{
    const int lane = threadIdx.x & 63;
    const int G1 = p.gamma + 1;
    // everything the outputs need, issued together: lane i <= gamma takes
    // position i's draft token and row statistics
    int32_t tok = 0;
    RowStat st{0.0f, 0, 0.0, 0.0, 0.0};
    if (lane <= p.gamma) {
        st = ld_stat(p.stats + (int64_t)b * G1 + lane);
        if (lane < p.gamma) tok = p.tokens[(int64_t)b * p.gamma + lane];
    }
    const uint64_t mask = ld_agent(&p.ctl[b].mask);
    const uint64_t merge_lost = ld_agent(&p.ctl[b].pad[0]);
    const double ug = (double)p.uniforms[(int64_t)b * G1 + p.gamma];
    const SubSum* ss = p.sub + (size_t)b * p.nsub;
    const int nrounds = (p.nsub + kRound - 1) / kRound;
    double rE[kRPL], rEA[kRPL], rQA[kRPL];
    bool marked = true;  // (MARKS) every sub-chunk of the rounds loaded so far has its done mark
    auto load_round = [&](int r) {
#pragma unroll
        for (int i = 0; i < kRPL; ++i) {
            const int j = r * kRound + lane * kRPL + i;
            if (j < p.nsub) {
                rE[i] = ld_agent_d(&ss[j].E);
                rEA[i] = ld_agent_d(&ss[j].EA);
                rQA[i] = ld_agent_d(&ss[j].QA);
                if constexpr (MARKS) marked = marked && ss[j].done != 0.0;
            } else {
                rE[i] = rEA[i] = rQA[i] = 0.0;
            }
        }
    };
    load_round(0);
    if constexpr (MARKS) {
        if (__ballot(!marked) != 0) return false;
    }

    const bool bad = __ballot(lane < p.gamma && (tok < 0 || tok >= p.V)) != 0;
    const int n = first_reject(mask, p.gamma);
    // a row on the walk whose merge ran out of its wait: the sequence is
    // reported like an invalid one, with n = -2, and counted
    const bool failed = (merge_lost & ((2ull << n) - 1ull)) != 0;
    const bool invalid = (mask & kInvalidBit) || bad || failed;
    const bool resid = n < p.gamma;
    int t = -1;
    double Z = NAN;
    double pout = NAN;  // p_n(t), when asked for
    if (!invalid) {
        // exact normaliser of row n and the residual mass
        double a = 0.0;
        for (int r = 0; r < nrounds; ++r) {
            if (r > 0) {
                load_round(r);
                if constexpr (MARKS) {
                    if (__ballot(!marked) != 0) return false;  // (no output written yet)
                }
            }
#pragma unroll
            for (int i = 0; i < kRPL; ++i) a += rE[i];
        }
        const double S = wave_sum_dpp(a);
        const double invS = 1.0 / S;  // p_v = e_v * invS (within an ulp of e_v / S)
        double zl = 0.0;
        if (resid) {
            for (int r = 0; r < nrounds; ++r) {
                if (nrounds > 1) load_round(r);
#pragma unroll
                for (int i = 0; i < kRPL; ++i) zl += fmax(0.0, rEA[i] * invS - p.len * rQA[i]);
            }
        }
        Z = wave_sum_dpp(zl);
        const bool use_resid = resid && Z > kResidEps;
        const double total = use_resid ? Z : S;
        const double target = ug * total;
        auto sub_weight = [&](int i) { return use_resid ? fmax(0.0, rEA[i] * invS - p.len * rQA[i]) : rE[i]; };

        // the sub-chunk whose running weight first exceeds the target: lane
        // totals scanned across the wave, then the crossing lane's entries
        int js = -1;
        double carry = 0.0, pre = 0.0;
        // u >= 1 puts u * total at the end of the row: no running sum exceeds
        // it, and the draw is the largest index with positive weight (below)
        for (int r = 0; r < nrounds && js < 0 && ug < 1.0; ++r) {
            if (nrounds > 1) load_round(r);
            double lt = 0.0;
#pragma unroll
            for (int i = 0; i < kRPL; ++i) lt += sub_weight(i);
            const double incl = wave_incl_scan_dpp(lt);
            double excl = __shfl_up(incl, 1, 64);
            if (lane == 0) excl = 0.0;
            const int L = first_lane(__ballot(lt > 0.0 && carry + incl > target));
            if (L >= 0) {
                int found = -1, ipos = -1;
                double c = carry + excl, cpos = c;
#pragma unroll
                for (int i = 0; i < kRPL; ++i) {
                    const double w = sub_weight(i);
                    if (found < 0 && w > 0.0) {
                        if (c + w > target) found = i;
                        else { ipos = i; cpos = c; c += w; }
                    }
                }
                if (found < 0) { found = ipos; c = cpos; }  // rounding: the lane's last positive entry
                const int f = __shfl(found, L, 64);
                pre = __shfl(c, L, 64);
                js = r * kRound + L * kRPL + f;
            } else {
                carry += __shfl(incl, 63, 64);
            }
        }

        // scan sub-chunk js a group (512 elements) at a time (and, only if
        // rounding pushed the crossing out of it, the groups after it) in
        // index order, every weight exact
        const int64_t row = (int64_t)b * G1 + n;
        const void* zrow = static_cast<const char*>(p.logits) + (size_t)row * p.V * (DT == SV_BF16 ? 2 : 4);
        const void* qrow = static_cast<const char*>(p.probs) +
                           (size_t)((int64_t)b * p.gamma + (resid ? n : 0)) * p.V * (PT == SV_BF16 ? 2 : 4);
        const double nMcd = -(double)__shfl(st.m, n, 64) * p.cd;  // lane n holds row n's statistics
        double rem = target - pre;
        int s_from = js * kSubPerWave;  // the first group the loop below scans
        if constexpr (PAR) {
            __shared__ double sm_tot[kWaves];
            __shared__ int sm_first, sm_t;
            const int w = (int)(threadIdx.x >> 6);
            if (js >= 0) {  // (uniform across the workgroup)
                const int s = js * kSubPerWave + w;
                const int idx = s * kSub + lane * 8;
                const bool have = s < p.nsub * kSubPerWave && s * kSub < p.V;
                Raw8 zr{}, qr{};
                if (have) {
                    zr = load_group<DT, VEC2>(zrow, idx, p.V);
                    if (use_resid) qr = load_group<PT, VEC2>(qrow, idx, p.V);
                }
                double wv[8], lt = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    wv[e] = have && idx + e < p.V ? draw_weight(p, use_resid, raw8_elem<DT>(zr, e),
                                                                use_resid ? raw8_elem<PT>(qr, e) : 0.0f, nMcd, invS)
                                                  : 0.0;
                    lt += wv[e];
                }
                const double incl = wave_incl_scan_dpp(lt);
                if (lane == 63) sm_tot[w] = incl;
                if (threadIdx.x == 0) sm_first = kWaves;
                __syncthreads();
                double rw = rem;  // the target less the groups before this one, subtracted in order
                for (int h = 0; h < w; ++h) rw -= sm_tot[h];
                const int L = first_lane(__ballot(have && lt > 0.0 && incl > rw));
                if (L >= 0 && lane == 0) atomicMin(&sm_first, w);
                __syncthreads();
                const int wf = sm_first;
                if (wf < kWaves) {
                    if (w == wf) {
                        double excl = __shfl_up(incl, 1, 64);
                        if (lane == 0) excl = 0.0;
                        int found = -1, ipos = -1;
                        double c = excl;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if (found < 0 && wv[e] > 0.0) {
                                if (c + wv[e] > rw) found = e;
                                else { ipos = e; c += wv[e]; }
                            }
                        }
                        if (found < 0) found = ipos;
                        const int tt = s * kSub + L * 8 + __shfl(found, L, 64);
                        if (lane == 0) sm_t = tt;
                    }
                    __syncthreads();
                    t = sm_t;
                } else {
                    // past the sub-chunk only by rounding: on from the next group
                    for (int h = 0; h < kWaves; ++h) rem -= sm_tot[h];
                    s_from = (js + 1) * kSubPerWave;
                }
            }
        }
        // the sub-chunk's groups, all loads in flight at once
        Raw8 zs[kSubPerWave], qs[kSubPerWave];
        if (!PAR && js >= 0) {
#pragma unroll
            for (int g = 0; g < kSubPerWave; ++g) {
                zs[g] = load_group<DT, VEC2>(zrow, (js * kSubPerWave + g) * kSub + lane * 8, p.V);
                if (use_resid) qs[g] = load_group<PT, VEC2>(qrow, (js * kSubPerWave + g) * kSub + lane * 8, p.V);
            }
        }
        for (int s = s_from; js >= 0 && s < p.nsub * kSubPerWave && t < 0; ++s) {
            const int idx = s * kSub + lane * 8;
            if (s * kSub >= p.V) break;
            const int g = s - js * kSubPerWave;
            Raw8 zr{}, qr{};
            if (!PAR && g < kSubPerWave) {
                // (a constant index into the prefetched groups)
#pragma unroll
                for (int h = 0; h < kSubPerWave; ++h)
                    if (h == g) { zr = zs[h]; qr = qs[h]; }
            } else {
                zr = load_group<DT, VEC2>(zrow, idx, p.V);
                if (use_resid) qr = load_group<PT, VEC2>(qrow, idx, p.V);
            }
            double w[8], lt = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                w[e] = idx + e < p.V ? draw_weight(p, use_resid, raw8_elem<DT>(zr, e),
                                                   use_resid ? raw8_elem<PT>(qr, e) : 0.0f, nMcd, invS)
                                     : 0.0;
                lt += w[e];
            }
            const double incl = wave_incl_scan_dpp(lt);
            double excl = __shfl_up(incl, 1, 64);
            if (lane == 0) excl = 0.0;
            const int L = first_lane(__ballot(lt > 0.0 && incl > rem));
            if (L >= 0) {
                int found = -1, ipos = -1;
                double c = excl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (found < 0 && w[e] > 0.0) {
                        if (c + w[e] > rem) found = e;
                        else { ipos = e; c += w[e]; }
                    }
                }
                if (found < 0) found = ipos;
                t = s * kSub + L * 8 + __shfl(found, L, 64);
            } else {
                rem -= __shfl(incl, 63, 64);
            }
        }
        if (t < 0) {
            // u * total at or past the end (only by rounding, u < 1): the
            // largest index with positive weight, searched backwards from the
            // last sub-chunk whose sum is positive
            int jl = -1;
            for (int r = 0; r < nrounds; ++r) {
                if (nrounds > 1) load_round(r);
#pragma unroll
                for (int i = 0; i < kRPL; ++i)
                    if (sub_weight(i) > 0.0) jl = r * kRound + lane * kRPL + i;
            }
            jl = wave_max_i(jl);
            auto scan_back = [&](int from, bool wres) {
                for (int s = from; s >= 0; --s) {
                    if (s * kSub >= p.V) continue;
                    const int idx = s * kSub + lane * 8;
                    const Raw8 zr = load_group<DT, VEC2>(zrow, idx, p.V);
                    Raw8 qr{};
                    if (wres) qr = load_group<PT, VEC2>(qrow, idx, p.V);
                    int lastv = -1;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (idx + e < p.V && draw_weight(p, wres, raw8_elem<DT>(zr, e),
                                                         wres ? raw8_elem<PT>(qr, e) : 0.0f, nMcd, invS) > 0.0)
                            lastv = idx + e;
                    lastv = wave_max_i(lastv);
                    if (lastv >= 0) return lastv;
                }
                return -1;
            };
            t = scan_back(jl * kSubPerWave + kSubPerWave - 1, use_resid);
            // (the residual support is chosen with the row stage's
            // normaliser; should no element of it survive the exact one, the
            // row n itself, which always has an element with e_v = 1)
            if (t < 0) t = scan_back(p.nsub * kSubPerWave - 1, false);
        }
        // p_n(t) = e_t / S, e_t by the draw's arithmetic
        if (p.aux_pout && t >= 0) pout = draw_weight(p, false, elem_at<DT>(zrow, t), 0.0f, nMcd, invS) * invS;
    }

    // outputs and telemetry
    if (PAR && threadIdx.x >= 64) return true;
    if (lane < G1) {
        int32_t o;
        if (invalid) o = -1;
        else if (lane < n) o = tok;
        else if (lane == n) o = t;
        else o = -1;
        p.tok_out[(int64_t)b * G1 + lane] = o;
        const bool row_seen = !invalid && lane <= n;
        if (p.aux_rmax) p.aux_rmax[(int64_t)b * G1 + lane] = row_seen ? st.m : NAN;
        if (p.aux_rsum) p.aux_rsum[(int64_t)b * G1 + lane] = row_seen ? st.S : NAN;
        if (lane < p.gamma) {
            if (p.aux_p) p.aux_p[(int64_t)b * p.gamma + lane] = row_seen ? st.P : NAN;
            if (p.aux_q) p.aux_q[(int64_t)b * p.gamma + lane] = row_seen ? st.Q : NAN;
        }
    }
    if (lane == 0) {
        if (failed && p.err_count) add_agent(p.err_count, 1u);
        p.n_out[b] = failed ? -2 : invalid ? -1 : n;
        if (p.aux_resid) p.aux_resid[b] = (!invalid && resid) ? Z : NAN;
        if (p.aux_pout) p.aux_pout[b] = pout;
    }
    return true;
}

// One claimed draw chunk of sequence b, by the whole workgroup: wave w takes
// sub-chunks c2 * 16 + 4w .. +3.  No workgroup barrier inside.  COUNTED:
// see draw_wave; returns true in the wave that completes the sequence.
template <int DT, int PT, bool VEC2, bool COUNTED>
__device__ __forceinline__ bool draw_chunk(const Params& p, int b, int c2, uint64_t mask, uint64_t target = 0)
{
    return draw_wave<DT, PT, VEC2, COUNTED>(p, b, wave_sub(c2, threadIdx.x >> 6) * kSubPerWave, mask, target);
}

// ------------------------------------------------------------ sample, launch 1

// Draw helpers, appended to the first launch's grid after every row block:
// helper j computes draw chunk j % nch2 of the sequence whose n became known
// (j / nch2)-th.  It waits, bounded, until that sequence is in the ready
// list; the entry carries b and n, and the sequence's reject bits and row n's
// statistics were published before it.  Being dispatched after every row
// block, the helpers take no slot from the rows of any position, and they
// wait only on row blocks, which never wait on them.  A helper whose wait
// runs out leaves its chunk to the last launch, which finds it by the sums'
// done marks.
template <int DT, int PT, bool VEC2>
__device__ void help_draw(const Params& p, int j)
{
    __shared__ uint32_t sm_he;
    __shared__ double sm_g[kWaves][3];
    const DrawTask task = p.fine ? fine_task(j, p.nsub) : helper_task(j, p.nch2);
    const int r = task.r;
    if (threadIdx.x == 0) {
        uint32_t e = 0;
        for (int it = 0; it < p.help_polls; ++it) {
            e = ld_agent32(&p.ready[r]);
            if (e != 0u) break;
            __builtin_amdgcn_s_sleep(8);
        }
        sm_he = e;
    }
    __syncthreads();
    const uint32_t e = sm_he;
    const int b = ready_seq(e), n = ready_n(e);
    if (e == 0u || b >= p.B || n > p.gamma) return;
    // (a mask with n's reject bit alone: the draw's row and residual follow from n)
    const uint64_t mask = n < p.gamma ? 1ull << n : 0ull;
    if (p.fine) {
        // sub-chunk task.c2, a group per wave, the group totals added in group order
        const int w = (int)(threadIdx.x >> 6);
        double E, EA, QA;
        draw_group<DT, PT, VEC2>(p, b, task.c2 * kSubPerWave + w, mask, E, EA, QA);
        if ((threadIdx.x & 63) == 0) {
            sm_g[w][0] = E;
            sm_g[w][1] = EA;
            sm_g[w][2] = QA;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            double e = 0.0, ea = 0.0, qa = 0.0;
            for (int i = 0; i < kWaves; ++i) {
                e += sm_g[i][0];
                ea += sm_g[i][1];
                qa += sm_g[i][2];
            }
            p.sub[(size_t)b * p.nsub + task.c2] = SubSum{e, ea, qa, 1.0};
        }
        return;
    }
    draw_chunk<DT, PT, VEC2, false>(p, b, task.c2, mask);
}

// Decision inputs read through the scalar cache: every lane of the workgroup
// asks for the same address and the inputs are read-only during the call.
// The scalar counter is separate from the vector one, so waiting for the
// control words or the chunk never waits for these, nor the other way round.
typedef const __attribute__((address_space(4))) uint32_t* ScalarU32;

__device__ __forceinline__ uint32_t scalar_word(const void* p)
{
    return *(ScalarU32)p;  // an address-space cast, which only a C-style cast can spell
}

// The aligned 32-bit word holding element idx (a workgroup-uniform index);
// word_elem() turns it into the element.  Kept apart so that the wait for the
// load falls where the value is used, not where it is loaded.
template <int DT>
__device__ __forceinline__ uint32_t scalar_elem_word(const void* base, int64_t idx, uint32_t& sel)
{
    if constexpr (DT == SV_FP32) {
        sel = 0;
        return scalar_word(static_cast<const float*>(base) + idx);
    } else {
        const uintptr_t a = reinterpret_cast<uintptr_t>(static_cast<const uint16_t*>(base) + idx);
        sel = (uint32_t)(a & 2) << 3;  // 16 for the high half
        return scalar_word(reinterpret_cast<const void*>(a & ~(uintptr_t)3));
    }
}

template <int DT>
__device__ __forceinline__ float word_elem(uint32_t w, uint32_t sel)
{
    if constexpr (DT == SV_FP32) return __uint_as_float(w);
    else return __uint_as_float((w >> sel) << 16);
}

// Draft token and uniform of position k of sequence b.
__device__ __forceinline__ void fetch_token_uniform(const Params& p, int b, int k, int& xk, float& uk)
{
    xk = (int)scalar_word(p.tokens + ((int64_t)b * p.gamma + k));
    uk = __uint_as_float(scalar_word(p.uniforms + ((int64_t)b * (p.gamma + 1) + k)));
}

// Scalar registers allowed to the first launch's kernel.  Measured on gfx950:
// a 256-thread workgroup at <= 64 VGPRs gets 8 waves per SIMD only while the
// kernel descriptor asks for at most ~78 SGPRs (7 at 86, 6 at 100), fewer
// than the compiler's occupancy model allows, so the cap is explicit (the
// few values it pushes out live in VGPR lanes).
constexpr int kMainSgprs = 80;

// VMODE: 0 scalar loads everywhere; 1 vector loads in the row stage only;
// 2 vector loads in the row stage and the draw.
template <int DT, int PT, int VMODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_num_sgpr(kMainSgprs))) void k_main_sample(const Params p)
{
    constexpr bool VEC = VMODE >= 1, VEC2 = VMODE == 2;
    constexpr int EPT = DT == SV_BF16 ? kEptBf16 : kEptFp32;
    constexpr int CH = EPT * kThreads;
    if (blockIdx.x >= (unsigned)p.rows_grid) {
        help_draw<DT, PT, VEC2>(p, (int)(blockIdx.x - (unsigned)p.rows_grid));
        return;
    }
    const RowBlock rb = row_block(blockIdx.x, p.nch1, p.B);
    const int c = rb.c, b = rb.b, k = rb.k;
    const int G1 = p.gamma + 1;
    const int64_t row = (int64_t)b * G1 + k;

    __shared__ float sm_f[kWaves];
    __shared__ int sm_i[kWaves];
    __shared__ double sm_d[kWaves];
    __shared__ int sm_cmd;

    // The decision inputs (draft token, uniform, then the token's logit and
    // draft probability) are fetched in case this block turns out to be the
    // row's last.  The token and uniform go out beside the control words (at
    // position 0, which has none, behind the chunk's loads); the two loads
    // that need the token go out behind the chunk's, so no dependent fetch
    // sits in front of the stream.
    int xk = 0;
    float uk = 0.0f;
    if (k > 0 && k < p.gamma) fetch_token_uniform(p, b, k, xk, uk);
    if (k > 0 && !p.tele) {
        // Is this row still needed?  Only a reject bit below k makes row k
        // unneeded.  A bad draft token at position j sets kInvalidBit
        // together with reject bit j, so rows past j skip while every row
        // before j is still streamed and decided: each position of the
        // sequence then gets a decision bit.
        if (threadIdx.x == 0) sm_cmd = (ld_agent(&p.ctl[b].mask) & ((1ull << k) - 1ull)) ? 1 : 0;
        __syncthreads();
        if (sm_cmd) return;
    }
    uint32_t zw = 0, qw = 0, zsel = 0, qsel = 0;
    uint32_t dep = 0;
    uint64_t evidence = 0, early_bit = 0;
    {
        const int v0 = c * CH;
        const void* rowp = static_cast<const char*>(p.logits) + (size_t)row * (size_t)p.V * (DT == SV_BF16 ? 2 : 4);
        ChunkRegs<DT, VEC, EPT> x;
        x.load(rowp, v0, p.V);
        if (k == 0 && p.gamma > 0) fetch_token_uniform(p, b, 0, xk, uk);
        if (k < p.gamma && xk >= 0 && xk < p.V) {
            zw = scalar_elem_word<DT>(p.logits, row * p.V + xk, zsel);
            qw = scalar_elem_word<PT>(p.probs, ((int64_t)b * p.gamma + k) * p.V + xk, qsel);
        }

        auto float_max = [&]() {
            float m = -INFINITY;
#pragma unroll
            for (int g = 0; g < EPT / 8; ++g) {
                float z[8];
                x.get8(g, z);
#pragma unroll
                for (int e = 0; e < 8; ++e) m = fmaxf(m, z[e]);
            }
            return block_max(m, sm_f);
        };
        float mx;
        if constexpr (DT == SV_BF16 && VEC) {
            const int hm = block_max_i(x.max_bits16(), sm_i);
            mx = hm >= 0 ? __uint_as_float((uint32_t)hm << 16) : float_max();
        } else {
            mx = float_max();
        }
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
            // the partial goes out with plain device-scope stores and the
            // count is taken at once; the row's last block waits until both
            // words of every slot have landed (neither written word is
            // zero: the max word carries a flag bit above the float, and
            // the sum, never negative, goes out with its sign bit flipped;
            // the two stores may land in either order)
            uint64_t* slot = p.part1 + 2 * ((size_t)row * p.nch1 + c);
            if (!(k == p.drop_slot && c == 0)) {
                st_agent(slot, (uint64_t)__float_as_uint(mx) | kSlotFlag);
                st_agent(slot + 1, dbits(s) ^ kSignBit);
            }
            if (k < p.gamma && xk >= 0 && xk < p.V) {
                evidence = rejection_evidence((double)uk, p.len * (double)word_elem<PT>(qw, qsel), s, mx,
                                              word_elem<DT>(zw, zsel), p.cd, p.ex);
                early_bit = 1ull << k;
            }
        }
    }

    if (!row_arrive(p, row, b, evidence, early_bit, dep)) return;

    // Last block of a fully processed row: wave 0 merges the chunk partials,
    // once every slot has landed (the stores were issued before the counts).
    const int lane = (int)threadIdx.x;
    float M = -INFINITY;
    double S = 0.0;
    float mj[kMaxSlotsPerLane];
    double sj[kMaxSlotsPerLane];
    bool lost = false;  // a slot that did not land within the bounded wait
    for (int j0 = 0; j0 < p.nch1; j0 += 64 * kMaxSlotsPerLane) {
#pragma unroll
        for (int r = 0; r < kMaxSlotsPerLane; ++r) {
            const int j = j0 + r * 64 + lane;
            uint64_t w0 = 0, w1 = 0;
            if (j < p.nch1) {
                const uint64_t* slot = p.part1 + 2 * ((size_t)row * p.nch1 + j);
                w0 = ld_agent(slot);
                w1 = ld_agent(slot + 1);
                for (int it = 0; (w0 == 0 || w1 == 0) && it < p.polls_slot; ++it) {
                    __builtin_amdgcn_s_sleep(1);
                    w0 = ld_agent(slot);
                    w1 = ld_agent(slot + 1);
                }
                if (w0 == 0 || w1 == 0) {
                    lost = true;
                    w0 = w1 = 0;
                }
            }
            mj[r] = j < p.nch1 && w0 != 0 ? __uint_as_float((uint32_t)w0) : -INFINITY;
            sj[r] = w1 != 0 ? __longlong_as_double((long long)(w1 ^ kSignBit)) : 0.0;
        }
        float mm = -INFINITY;
#pragma unroll
        for (int r = 0; r < kMaxSlotsPerLane; ++r) mm = fmaxf(mm, mj[r]);
        mm = wave_max(mm);
        // rescale what is merged so far to the new maximum
        if (mm > M) {
            if (M > -INFINITY) S *= exp2_f64(((double)M - (double)mm) * p.cd, p.ex);
            M = mm;
        }
#pragma unroll
        for (int r = 0; r < kMaxSlotsPerLane; ++r)
            if (mj[r] > -INFINITY) S += sj[r] * exp2_f64(((double)mj[r] - (double)M) * p.cd, p.ex);
    }
    S = wave_sum(S);
    const bool failed = __ballot(lost) != 0;

    if (threadIdx.x == 0) {
        double P = NAN, Q = NAN;
        uint64_t maskbits = 0;
        if (k < p.gamma) {
            // [FI] Phase 3 / [PB] section 3: accept x_k iff u_k <= min(1, p/q),
            // q <= 0 accepts ([PB] Reference Implementation); with a lenience
            // l, q is scaled by l first ([FI] Appendix A.5).
            if (xk < 0 || xk >= p.V) {
                maskbits = kInvalidBit | (1ull << k);
            } else {
                P = exp2(((double)word_elem<DT>(zw, zsel) - (double)M) * p.cd) / S;
                Q = (double)word_elem<PT>(qw, qsel);
                const double thr = Q <= 0.0 ? 1.0 : fmin(1.0, P / (p.len * Q));
                if (!((double)uk <= thr)) maskbits = 1ull << k;
            }
        }
        // the failure mark (its sequence's outputs are withheld), the
        // statistics, then the reject bit, then the decision bit that
        // announces them (a rejection decides every later position too)
        uint64_t dd = 0;
        if (failed) dd ^= or_agent(&p.ctl[b].pad[0], 1ull << k);
        const uint64_t w[4] = {stat_word0(M, -1), dbits(S), dbits(P), dbits(Q)};
        dd ^= publish(reinterpret_cast<uint64_t*>(p.stats + row), w, p.zero);
        if (maskbits) dd ^= or_agent(&p.ctl[b].mask, maskbits) & p.zero;
        const uint64_t all = rows_mask(p.gamma);
        const uint64_t decbits = maskbits ? (all & ~((1ull << k) - 1ull)) : (1ull << k);
        const uint64_t old = or_agent(&p.ctl[b].dec, decbits | (uint64_t)(fold64(dd) & p.zero));
        if ((old & all) != all && ((old | decbits) & all) == all) {
            // n of this sequence just became known: record the order, with n
            // (read by the draw helpers and the last launch).  Every position
            // before k was decided and accepted (a rejection there would have
            // set bit k already), so a rejection here makes n = k, and the
            // bonus row's block completing the mask makes n = gamma.  Else
            // n > k is the first reject bit of the mask, read once dec has
            // returned: that rejection was performed before its decision
            // bits, which this block saw.
            int n = maskbits ? k : p.gamma;
            if (!maskbits && k < p.gamma)
                n = first_reject(ld_agent(&p.ctl[b].mask + (fold64(old) & p.zero)), p.gamma);
            const uint32_t slot = add_agent(p.ready_cnt, 1u);
            const uint32_t e = ((uint32_t)b + 1u) | ((uint32_t)n << kReadyNShift);
            __hip_atomic_store(&p.ready[slot], e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            or_agent(&p.ctl[b].retire, (uint64_t)slot << 32);
        }
    }
}

// ------------------------------------------------------- acceptance telemetry

// beta of position i of sequence b: sum_v min(p_i(v), q_i(v)) ("Fast
// Inference from Transformers via Speculative Decoding", summary page,
// Theorem 3.5), swept after the first launch, which in telemetry mode
// leaves the statistics of every row.  One workgroup per kChunkB elements
// of row (b, i): p_v = 2^((z_v - m) log2(e)/T) / S with the fp32 exp2 of the
// row stage (the shift's rounding eta folded into the scale), q_v exact,
// min and sum in fp64; the workgroup's sum goes to its slot, and
// k_beta_merge adds a row's slots in index order.
template <int DT, int PT, bool VEC2>
__global__ __launch_bounds__(kThreads) void k_beta(const Params p)
{
    const BetaBlock bb = beta_block(blockIdx.x, p.nchb, p.gamma);
    const int c = bb.c, b = bb.b, i = bb.i;
    const int t = b * p.gamma + i;
    const int64_t row = (int64_t)b * (p.gamma + 1) + i;
    __shared__ double sm_d[kWaves];
    const int tid = (int)threadIdx.x;

    const void* zrow = static_cast<const char*>(p.logits) + (size_t)row * p.V * (DT == SV_BF16 ? 2 : 4);
    const void* qrow = static_cast<const char*>(p.probs) + (size_t)t * p.V * (PT == SV_BF16 ? 2 : 4);
    Raw8 zr[kGroupsB], qr[kGroupsB];
#pragma unroll
    for (int g = 0; g < kGroupsB; ++g) {
        const int idx = c * kChunkB + (g * kThreads + tid) * 8;
        zr[g] = load_group<DT, VEC2>(zrow, idx, p.V);
        qr[g] = load_group<PT, VEC2>(qrow, idx, p.V);
    }
    const uint64_t* sw = reinterpret_cast<const uint64_t*>(p.stats + row);
    const double mc = (double)__uint_as_float((uint32_t)ld_agent(sw)) * p.cd;
    const double S = __longlong_as_double((long long)ld_agent(sw + 1));
    const float K = (float)(-mc);
    // p_v = 2^(...) * scale in fp32 (the row stage's exponential, ~3e-7
    // relative), min(p_v, q_v) in fp32, eight at a time into an fp64 sum:
    // beta is reported to 1e-6 absolute
    const float scale = (float)(exp2(-((double)K + mc)) / S);
    const bool full = (c + 1) * kChunkB <= p.V;  // (uniform) no entry of the chunk past the row

    double acc = 0.0;
#pragma unroll
    for (int g = 0; g < kGroupsB; ++g) {
        const int idx = c * kChunkB + (g * kThreads + tid) * 8;
        float m8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float z = raw8_elem<DT>(zr[g], e);
            const float pv = __builtin_amdgcn_exp2f(fmaf(z, p.c_lo, fmaf(z, p.c_hi, K))) * scale;
            m8[e] = fminf(pv, raw8_elem<PT>(qr[g], e));
            if (!full && idx + e >= p.V) m8[e] = 0.0f;
        }
        acc += (double)(((m8[0] + m8[1]) + (m8[2] + m8[3])) + ((m8[4] + m8[5]) + (m8[6] + m8[7])));
    }
    const double s = block_sum(acc, sm_d);
    if (tid == 0) p.bpart[(size_t)t * p.nchb + c] = s;

    // The draw of a sequence rejected at position i reads these same two
    // rows: its draw chunk c (the same span of the row) is summed here and
    // counted as claimed, so the last launch only finishes the draw.  (The
    // first launch, which streamed every row, has claimed nothing.)
    const uint64_t mask = ld_agent(&p.ctl[b].mask);
    if (!(mask & kInvalidBit) && first_reject(mask, p.gamma) == i) {
        draw_chunk<DT, PT, VEC2, false>(p, b, c, mask);
        if (tid == 0) add_agent64(&p.ctl[b].claim, 1ull);
    }
}

// beta[b][i] = the row's slots added in index order (and cleared); alpha[i]
// = the mean over b, with a fixed reduction tree.  One workgroup per
// position.
__global__ __launch_bounds__(kThreads) void k_beta_merge(const Params p)
{
    const int i = (int)blockIdx.x;
    __shared__ double sm_d[kWaves];
    double a = 0.0;
    for (int b = (int)threadIdx.x; b < p.B; b += kThreads) {
        double* slot = p.bpart + ((size_t)b * p.gamma + i) * p.nchb;
        double s = 0.0;
#pragma unroll 4
        for (int c = 0; c < p.nchb; ++c) {
            s += slot[c];
            slot[c] = 0.0;
        }
        if (p.aux_beta) p.aux_beta[(int64_t)b * p.gamma + i] = s;
        a += s;
    }
    a = block_sum(a, sm_d);
    if (threadIdx.x == 0 && p.aux_alpha) p.aux_alpha[i] = a / (double)p.B;
}

// ------------------------------------------------------------ sample, launch 2

// The last launch of telemetry calls, nch2 workgroups per sequence.  The
// telemetry sweep took draw chunks 0 .. L1-1 of a sequence (its claim count,
// final now: the sweep's workgroups of the rejected row n sum them); chunk L1 + j
// goes to the sequence's workgroup j, and a workgroup with no chunk left
// returns after reading that count.  Workgroup i < B is workgroup 0 of the
// sequence whose n became known (B-1-i)-th; the others (nch2 - 1 per
// sequence) follow in the same order, so the sequences resolved last, which
// have the most chunks left, are served first.  The wave that completes the
// sequence's remaining wave tasks (workgroup 0 itself when none is left) runs
// the draw; the last of the sequence's users here (its workgroups with a
// chunk, and the draw) clears its workspace.
template <int DT, int PT, bool VEC2>
__global__ __launch_bounds__(kThreads) void k_rest_sample(const Params p)
{
    const RestTask rt = rest_task((int)blockIdx.x, p.B, p.nch2);
    const int r = rt.r, j = rt.j;
    // (every sequence is in the list once launch 1 is done, and leaves it when
    // the last of its users here clears its workspace)
    const uint32_t listed = ld_agent32(&p.ready[r]);
    const int b = ready_seq(listed);
    if (listed == 0u || b >= p.B) return;
    // the first launch's claim count, final during this launch -- unless the
    // sequence has been cleared meanwhile, in which case it is no longer
    // listed and this workgroup had nothing to do
    const uint64_t claim = ld_agent(&p.ctl[b].claim);
    const uint64_t mask = ld_agent(&p.ctl[b].mask);  // final too: the row stage has finished
    if (ld_agent32(&p.ready[r] + (fold64(claim ^ mask) & p.zero)) != listed) return;
    const int l1 = (int)min((uint32_t)claim, (uint32_t)p.nch2);
    const int left = p.nch2 - l1;
    const int users = max(left, 1);  // workgroups of the sequence with work here
    if (j >= users) return;
    bool fin_wave = false;
    if (left == 0) fin_wave = threadIdx.x < 64;  // nothing left: workgroup 0 draws
    else if (draw_chunk<DT, PT, VEC2, true>(p, b, l1 + j, mask, (uint64_t)kWaves * left)) fin_wave = true;
    if (fin_wave) {
        finish_wave<DT, PT, VEC2, false>(p, b);
        retire_wave(p, b, (uint32_t)users + 1u);
    }
    __syncthreads();  // this workgroup's work is done
    if (threadIdx.x < 64) retire_wave(p, b, (uint32_t)users + 1u);
}

// The last launch when the first launch carries draw helpers: workgroup b
// finishes sequence b.  Its waves run the draw from the helpers' sums; should a
// sub-chunk lack its done mark (its helper's wait ran out), the workgroup
// computes every unmarked sub-chunk, counting them out, and the wave that
// completes the count runs the draw.  Then the sequence is cleared.  The
// first launch is over, so plain loads see its writes, and no other
// workgroup reads this sequence's workspace.
template <int DT, int PT, bool VEC2>
__global__ __launch_bounds__(kThreads) void k_finish_sample(const Params p)
{
    __shared__ int sm_ok, sm_left;
    const int b = (int)blockIdx.x;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // (every sequence is decided, and listed, in the first launch: the
    // decider of each position up to the first rejection takes part)
    const uint32_t rank = (uint32_t)(p.ctl[b].retire >> 32);  // its place in the ready list
    {
        // every wave (the four groups of the chosen sub-chunk are scanned side
        // by side); each returns the same result
        const bool ok = finish_wave<DT, PT, VEC2, true, true>(p, b);
        if (threadIdx.x == 0) sm_ok = ok ? 1 : 0;
    }
    if (threadIdx.x == 0) sm_left = 0;
    __syncthreads();
    if (!sm_ok) {
        const uint64_t mask = p.ctl[b].mask;
        const SubSum* ss = p.sub + (size_t)b * p.nsub;
        // sub-chunks left: wave w looks at w, w + 4, ... (lane i at the i-th of them)
        int mine = 0;
        for (int s0 = w; s0 < p.nsub; s0 += kWaves * 64) {
            const int sidx = s0 + kWaves * lane;
            mine += __popcll(__ballot(sidx < p.nsub && ss[sidx].done == 0.0));
        }
        if (lane == 0 && mine) atomicAdd(&sm_left, mine);
        __syncthreads();
        const int left = sm_left;
        bool fin_wave = false;
        for (int s0 = w; s0 < p.nsub; s0 += kWaves * 64) {
            const int sidx = s0 + kWaves * lane;
            uint64_t todo = __ballot(sidx < p.nsub && ss[sidx].done == 0.0);
            while (todo) {
                const int i = __builtin_ctzll(todo);
                todo &= todo - 1ull;
                if (draw_wave<DT, PT, VEC2, true>(p, b, (s0 + kWaves * i) * kSubPerWave, mask, (uint64_t)left))
                    fin_wave = true;
            }
        }
        if (fin_wave) finish_wave<DT, PT, VEC2, false>(p, b);
    }
    __syncthreads();  // the draw's reads are done
    if (w == 0) cleanup_wave(p, b, rank, true, false);
}

// ----------------------------------------------------------------- greedy mode

__device__ __forceinline__ bool greedy_skipped(const Params& p, int b, int k, int* sm_flag)
{
    if (k == 0) return false;  // position 0 is always needed (k is uniform)
    if (threadIdx.x == 0) {
        // (a bad token at position j also sets reject bit j: see k_main_sample)
        const uint64_t m = ld_agent(&p.ctl[b].mask);
        *sm_flag = (m & ((1ull << k) - 1ull)) ? 1 : 0;
    }
    __syncthreads();
    return *sm_flag != 0;
}

// EPT: entries per thread (kEptBf16 or kEptFp32; for bf16 rows of small
// batches kEptFp32, so half-size chunks, see make_plan).
template <int DT, bool VEC, int EPT>
__global__ __launch_bounds__(kThreads) void k_rows_greedy(const Params p)
{
    constexpr int W = DT == SV_BF16 ? 8 : 4;
    constexpr int CH = EPT * kThreads;
    const RowBlock rb = row_block(blockIdx.x, p.nch1, p.B);
    const int c = rb.c, b = rb.b, k = rb.k;
    const int G1 = p.gamma + 1;
    const int64_t row = (int64_t)b * G1 + k;

    __shared__ float sm_f[kWaves];
    __shared__ int sm_i[kWaves];
    __shared__ int sm_flag;

    if (greedy_skipped(p, b, k, &sm_flag)) return;
    // the draft token and its logit, for an early rejection by this chunk
    int xk = -1;
    float zx = 0.0f;
    if (threadIdx.x == 0 && k < p.gamma) {
        xk = p.tokens[(int64_t)b * p.gamma + k];
        if (xk >= 0 && xk < p.V) zx = load_one<DT>(p.logits, row * p.V + xk);
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
            dep = publish(p.part1 + 2 * ((size_t)row * p.nch1 + c), w, p.zero);
            // an element of this chunk beats the draft token for the argmax
            // (larger, or equal at a lower index): the position is rejected
            if (k < p.gamma && xk >= 0 && xk < p.V && bi != INT_MAX && (bv > zx || (bv == zx && bi < xk)))
                or_agent(&p.ctl[b].mask, 1ull << k);
        }
    }

    if (!row_arrive(p, row, b, 0, 0, dep)) return;

    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int j = (int)threadIdx.x; j < p.nch1; j += 64) {
        const uint64_t w = ld_agent(p.part1 + 2 * ((size_t)row * p.nch1 + j));
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
            if (bits) or_agent(&p.ctl[b].mask, bits);
        }
        p.stats[row] = st;  // read by the next launch
    }
}

__global__ __launch_bounds__(kThreads) void k_draw_greedy(const Params p)
{
    // one wave per sequence: n is the first rejected position, the token the
    // argmax of row n ([FI] "Standardized Sampling", argmax case)
    const int b = blockIdx.x;
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    const int G1 = p.gamma + 1;
    const uint64_t m = p.ctl[b].mask;
    const int n = first_reject(m, p.gamma);
    int32_t tok = 0;
    RowStat st{0.0f, 0, 0.0, 0.0, 0.0};
    if (lane <= p.gamma) {
        st = p.stats[(int64_t)b * G1 + lane];
        if (lane < p.gamma) tok = p.tokens[(int64_t)b * p.gamma + lane];
    }
    const bool bad = __ballot(lane < p.gamma && (tok < 0 || tok >= p.V)) != 0;
    const bool invalid = (m & kInvalidBit) || bad;
    const int t = __shfl(st.amax, min(n, 63), 64);
    if (lane < G1) {
        int32_t o;
        if (invalid) o = -1;
        else if (lane < n) o = tok;
        else if (lane == n) o = t;
        else o = -1;
        p.tok_out[(int64_t)b * G1 + lane] = o;
        const bool row_seen = !invalid && lane <= n;
        if (p.aux_rmax) p.aux_rmax[(int64_t)b * G1 + lane] = row_seen ? st.m : NAN;
        if (p.aux_rsum) p.aux_rsum[(int64_t)b * G1 + lane] = NAN;
        if (lane < p.gamma) {
            if (p.aux_p) p.aux_p[(int64_t)b * p.gamma + lane] = NAN;
            if (p.aux_q) p.aux_q[(int64_t)b * p.gamma + lane] = NAN;
        }
    }
    if (lane == 0) {
        p.n_out[b] = invalid ? -1 : n;
        if (p.aux_resid) p.aux_resid[b] = NAN;
        if (p.aux_pout) p.aux_pout[b] = NAN;
    }
    cleanup_wave(p, b, 0u, false);  // (no ready list in greedy mode)
}

__global__ void k_fill_zero(uint4* p, size_t n16, unsigned char* tail, size_t ntail)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
    if (i < ntail) tail[i] = 0;
}

// ------------------------------------------------------- small vocabularies

// Rows of at most kSmallV entries: one wave verifies a whole sequence in a
// single launch -- row statistics, the acceptance walk, the draw and the
// outputs ([FI] Algorithm 1, Phases 3 and 4; [PB] section 3; [ST]) -- with
// entry v of a row in lane v % 64, register v / 64, so a row is one
// coalesced load per register and index order is (register, lane).  Every
// e_v = 2^((z_v - m) log2(e)/T) is fp64 here, so S and p(x) are exact to
// rounding.  The many-workgroup path above would spend a workgroup per row
// chunk on a few entries.  Telemetry calls take that path.
constexpr int kSmallK = 8;              // entries per lane
constexpr int kSmallV = 64 * kSmallK;   // 512

// max / min over the wave with DPP moves and four row read-outs (see
// wave_sum_dpp)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_max_dpp(float v)
{
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ int wave_min_i_dpp(int v)
{
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

template <int DT, int PT, bool GREEDY>
__global__ __launch_bounds__(kThreads) void k_small(const Params p)
{
    const int lane = threadIdx.x & 63;
    const int b = (int)(blockIdx.x * kWaves + (threadIdx.x >> 6));
    if (b >= p.B) return;  // a whole wave: there is no barrier in this kernel
    const int G1 = p.gamma + 1;
    const int V = p.V;
    const int KV = (V + 63) / 64;  // registers that hold entries (wave-uniform): the rest is skipped
    int32_t tok = 0;
    float ul = 0.0f;
    if (lane < p.gamma) tok = p.tokens[(int64_t)b * p.gamma + lane];
    if (!GREEDY && lane < G1) ul = p.uniforms[(int64_t)b * G1 + lane];
    const bool invalid = __ballot(lane < p.gamma && (tok < 0 || tok >= V)) != 0;

    // lane i keeps row i's statistics for the outputs
    float st_m = NAN;
    double st_S = NAN, st_P = NAN, st_Q = NAN;
    int n = p.gamma, t = -1;
    double Z = NAN, pout = NAN;
    if (!invalid) {
        float z[kSmallK];
        double e[kSmallK];
        double S = 0.0;
        for (int i = 0; i <= p.gamma; ++i) {
            const void* zrow = static_cast<const char*>(p.logits) +
                               (size_t)((int64_t)b * G1 + i) * V * (DT == SV_BF16 ? 2 : 4);
            float m = -INFINITY;
#pragma unroll
            for (int j = 0; j < kSmallK; ++j) {
                const int v = lane + 64 * j;
                z[j] = j < KV && v < V ? elem_at<DT>(zrow, v) : -INFINITY;
                m = fmaxf(m, z[j]);
            }
            m = wave_max_dpp(m);
            if (lane == i) st_m = m;
            if constexpr (GREEDY) {
                // [FI] "Standardized Sampling", argmax case: the first index
                // attaining the maximum; the draft survives iff it is that index
                int a = INT_MAX;
#pragma unroll
                for (int j = kSmallK - 1; j >= 0; --j)
                    if (j < KV && lane + 64 * j < V && z[j] == m) a = lane + 64 * j;
                a = wave_min_i_dpp(a);
                if (i == p.gamma || __shfl(tok, i, 64) != a) {
                    n = i;
                    t = a;
                    break;
                }
            } else {
                const double nMcd = -(double)m * p.cd;
                double es = 0.0;
#pragma unroll
                for (int j = 0; j < kSmallK; ++j) {
                    e[j] = 0.0;
                    if (j < KV) {
                        if (lane + 64 * j < V) e[j] = exp2_f64(fma((double)z[j], p.cd, nMcd), p.ex);
                        es += e[j];
                    }
                }
                S = wave_sum_dpp(es);
                if (lane == i) st_S = S;
                if (i == p.gamma) break;  // every draft accepted: row gamma is the bonus row
                const int x = __shfl(tok, i, 64);
                const float zx = elem_at<DT>(zrow, x);
                const double P = zx > -INFINITY ? exp2(((double)zx - (double)m) * p.cd) / S : 0.0;
                const void* qrow = static_cast<const char*>(p.probs) +
                                   (size_t)((int64_t)b * p.gamma + i) * V * (PT == SV_BF16 ? 2 : 4);
                const double Q = (double)elem_at<PT>(qrow, x);
                if (lane == i) { st_P = P; st_Q = Q; }
                // accept iff u <= min(1, p / q), q scaled by the lenience; q <= 0 accepts
                const double thr = Q <= 0.0 ? 1.0 : fmin(1.0, P / (p.len * Q));
                if (!((double)__shfl(ul, i, 64) <= thr)) {
                    n = i;
                    break;
                }
            }
        }
        if constexpr (!GREEDY) {
            // the draw from row n (e and S of that row are in registers):
            // norm(max(0, p - l q)) after a rejection, p itself when that mass
            // is at most 1e-15 or every draft was accepted
            const bool resid = n < p.gamma;
            const double invS = 1.0 / S;
            double w[kSmallK];
            if (resid) {
                const void* qrow = static_cast<const char*>(p.probs) +
                                   (size_t)((int64_t)b * p.gamma + n) * V * (PT == SV_BF16 ? 2 : 4);
                double zs = 0.0;
#pragma unroll
                for (int j = 0; j < kSmallK; ++j) {
                    const int v = lane + 64 * j;
                    w[j] = 0.0;
                    if (j < KV) {
                        if (v < V) w[j] = fmax(0.0, e[j] * invS - p.len * (double)elem_at<PT>(qrow, v));
                        zs += w[j];
                    }
                }
                Z = wave_sum_dpp(zs);
            }
            const bool use_resid = resid && Z > kResidEps;
            if (!use_resid) {
#pragma unroll
                for (int j = 0; j < kSmallK; ++j) w[j] = e[j];
            }
            const double target = (double)__shfl(ul, p.gamma, 64) * (use_resid ? Z : S);
            // smallest index whose running weight (index order) exceeds the target
            double carry = 0.0;
#pragma unroll
            for (int j = 0; j < kSmallK; ++j) {
                if (t >= 0 || j >= KV) break;
                const double incl = wave_incl_scan_dpp(w[j]);
                const int L = first_lane(__ballot(w[j] > 0.0 && carry + incl > target));
                if (L >= 0) t = L + 64 * j;
                else carry += __shfl(incl, 63, 64);
            }
            if (t < 0) {
                // u * total at or past the end (only by rounding): the last positive weight
                int last = -1;
#pragma unroll
                for (int j = 0; j < kSmallK; ++j)
                    if (w[j] > 0.0) last = lane + 64 * j;
                t = wave_max_i(last);
            }
            if (!resid) Z = NAN;
            // p_n(t) = e_t / S: e and S of row n are in registers
            if (p.aux_pout && t >= 0) {
                double et = 0.0;
#pragma unroll
                for (int j = 0; j < kSmallK; ++j)
                    if (j == t / 64) et = e[j];
                pout = __shfl(et, t % 64, 64) * invS;
            }
        }
    }

    if (lane < G1) {
        int32_t o;
        if (invalid) o = -1;
        else if (lane < n) o = tok;
        else if (lane == n) o = t;
        else o = -1;
        p.tok_out[(int64_t)b * G1 + lane] = o;
        const bool row_seen = !invalid && lane <= n;
        if (p.aux_rmax) p.aux_rmax[(int64_t)b * G1 + lane] = row_seen ? st_m : NAN;
        if (p.aux_rsum) p.aux_rsum[(int64_t)b * G1 + lane] = row_seen && !GREEDY ? st_S : NAN;
        if (lane < p.gamma) {
            if (p.aux_p) p.aux_p[(int64_t)b * p.gamma + lane] = row_seen && !GREEDY ? st_P : NAN;
            if (p.aux_q) p.aux_q[(int64_t)b * p.gamma + lane] = row_seen && !GREEDY ? st_Q : NAN;
        }
    }
    if (lane == 0) {
        p.n_out[b] = invalid ? -1 : n;
        if (p.aux_resid) p.aux_resid[b] = invalid || GREEDY ? NAN : Z;
        if (p.aux_pout) p.aux_pout[b] = invalid || GREEDY ? NAN : pout;
    }
}

// Rows of at most 16 entries with gamma < 16 (c1: V = 8): one 16-lane DPP row
// per sequence, four sequences per wave; entry v in lane v of the row.  The
// same steps as k_small, with every reduction and scan kept inside the row
// (quad swaps and mirrors, row_shr), and the four walks run in lockstep with
// every lane active, each row masked once its walk has ended.
constexpr int kTinyV = 16;

// Reductions and scans inside rows of RL = 8 or 16 lanes: quad swaps, the
// half-row mirror (8 lanes), the row mirror (16); row_shr for the scan, with
// the shifts that would cross an 8-lane segment masked off.
template <int RL>
__device__ __forceinline__ float row_max(float v)
{
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    if constexpr (RL == 16) v = fmaxf(v, dpp_f<0x140>(v));
    return v;
}
template <int RL>
__device__ __forceinline__ int row_min(int v)
{
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false));
    if constexpr (RL == 16) v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false));
    return v;
}
template <int RL>
__device__ __forceinline__ double row_sum(double v)
{
    v += dpp_d<0xB1>(v);
    v += dpp_d<0x4E>(v);
    v += dpp_d<0x141>(v);
    if constexpr (RL == 16) v += dpp_d<0x140>(v);
    return v;
}
template <int RL>
__device__ __forceinline__ double row_incl_scan(double v)
{
    if constexpr (RL == 16) {
        v += dpp_d<0x111>(v);
        v += dpp_d<0x112>(v);
        v += dpp_d<0x114>(v);
        return v + dpp_d<0x118>(v);
    } else {
        const int l = (int)threadIdx.x & 7;
        double t = dpp_d<0x111>(v);
        v += l >= 1 ? t : 0.0;
        t = dpp_d<0x112>(v);
        v += l >= 2 ? t : 0.0;
        t = dpp_d<0x114>(v);
        return v + (l >= 4 ? t : 0.0);
    }
}

template <int DT, int PT, bool GREEDY, int TG, int RL>
__global__ __launch_bounds__(kThreads) void k_tiny(const Params p)
{
    constexpr int RPW = 64 / RL;  // rows (sequences) per wave
    const int lane = threadIdx.x & 63;
    const int r = lane / RL, l = lane % RL;  // row (sequence) of the wave, lane in the row
    const int b = (int)((blockIdx.x * kWaves + (threadIdx.x >> 6)) * RPW) + r;
    const bool live = b < p.B;  // rows past the batch run along masked (no loads, no stores)
    const int G1 = p.gamma + 1;
    const int V = p.V;
    const int base = lane & ~(RL - 1);
    constexpr uint64_t kRowBits = RL == 16 ? 0xffffull : 0xffull;
    int32_t tok = 0;
    float ul = 0.0f;
    if (live && l < p.gamma) tok = p.tokens[(int64_t)b * p.gamma + l];
    if (!GREEDY && live && l < G1) ul = p.uniforms[(int64_t)b * G1 + l];
    // every target row of the sequence (gamma + 1 <= TG) in registers,
    // loaded in one round trip with the tokens and uniforms: zs[i] = z_i(l)
    float zs[TG];
#pragma unroll
    for (int i = 0; i < TG; ++i) {
        zs[i] = -INFINITY;
        if (i <= p.gamma && live && l < V)
            zs[i] = elem_at<DT>(static_cast<const char*>(p.logits) +
                                    (size_t)((int64_t)b * G1 + i) * V * (DT == SV_BF16 ? 2 : 4), l);
    }
    const uint64_t bad = __ballot(live && l < p.gamma && (tok < 0 || tok >= V));
    const bool invalid = ((bad >> (RL * r)) & kRowBits) != 0ull;
    // lane i of a row: q_i(x_i), gathered once the tokens are in
    float qx = 0.0f;
    if (!GREEDY && live && !invalid && l < p.gamma)
        qx = elem_at<PT>(static_cast<const char*>(p.probs) + (size_t)((int64_t)b * p.gamma + l) * V * (PT == SV_BF16 ? 2 : 4),
                         tok);

    float st_m = NAN;
    double st_S = NAN, st_P = NAN, st_Q = NAN;
    int n = p.gamma, t = -1;
    double Z = NAN, pout = NAN;
    bool active = live && !invalid;  // this row's walk goes on
    double e = 0.0, S = 0.0;
    float z = -INFINITY;
#pragma unroll 1
    for (int i = 0; i <= p.gamma; ++i) {
        if (__ballot(active) == 0ull) break;
        z = active && l < V ? zs[i] : -INFINITY;  // (i is uniform: the arrays stay in registers)
        const float m = row_max<RL>(z);
        if (active && l == i) st_m = m;
        if constexpr (GREEDY) {
            const int a = row_min<RL>(l < V && z == m ? l : INT_MAX);
            const bool stop = i == p.gamma || __shfl(tok, base + i, 64) != a;
            if (active && stop) {
                n = i;
                t = a;
                active = false;
            }
        } else {
            // e and S keep row n's values once a row's walk has ended
            const double ei = active && l < V ? exp2_f64(fma((double)z, p.cd, -(double)m * p.cd), p.ex) : 0.0;
            const double Si = row_sum<RL>(ei);
            if (active) { e = ei; S = Si; }
            if (active && l == i) st_S = Si;
            if (i == p.gamma) break;  // the rows still walking accepted every draft
            const int x = __shfl(tok, base + i, 64);
            const double ex = __shfl(ei, base + (x & (RL - 1)), 64);  // e_x: lane x of the row holds it (x < V <= RL)
            const float ui = __shfl(ul, base + i, 64);
            double Q = 0.0;
            bool rej = false;
            const float qi = __shfl(qx, base + i, 64);  // q_i(x_i)
            if (active) {
                Q = (double)qi;
                // u <= min(1, p / (l q)) with p = e_x / S_i, q <= 0 accepting,
                // without divisions: for u <= 1 the same as q <= 0 or
                // u l q S_i <= e_x (rounding can differ only within the
                // flagged window)
                rej = !((double)ui <= 1.0 && (Q <= 0.0 || (double)ui * (p.len * Q) * Si <= ex));
            }
            if (active && l == i) { st_P = ex; st_Q = Q; }  // (e_x here: p_i(x_i) = e_x / S_i at the output)
            if (active && rej) {
                n = i;
                active = false;
            }
        }
    }
    if constexpr (!GREEDY) {
        // the draw of every row that walked (n and its e, S are this row's)
        const bool walked = live && !invalid;
        const bool resid = n < p.gamma;
        double w = e;
        double Zr = 0.0;
        if (walked && resid) {
            const void* qrow = static_cast<const char*>(p.probs) +
                               (size_t)((int64_t)b * p.gamma + n) * V * (PT == SV_BF16 ? 2 : 4);
            const double q = l < V ? (double)elem_at<PT>(qrow, l) : 0.0;
            w = l < V ? fmax(0.0, e * (1.0 / S) - p.len * q) : 0.0;
        }
        if (!(walked && resid)) w = walked ? e : 0.0;
        Zr = row_sum<RL>(walked && resid ? w : 0.0);
        const bool use_resid = walked && resid && Zr > kResidEps;
        if (walked && resid && !use_resid) w = e;
        const double total = use_resid ? Zr : S;
        const double target = (double)__shfl(ul, base + p.gamma, 64) * total;
        const double incl = row_incl_scan<RL>(w);
        const uint64_t hit = __ballot(walked && w > 0.0 && incl > target);
        const uint32_t hr = (uint32_t)((hit >> (RL * r)) & kRowBits);
        const uint64_t pos = __ballot(walked && w > 0.0);
        const uint32_t pr = (uint32_t)((pos >> (RL * r)) & kRowBits);
        if (walked) t = hr ? __builtin_ctz(hr) : (pr ? 31 - __builtin_clz(pr) : -1);
        if (walked && resid) Z = Zr;
        // p_n(t) = e_t / S: lane t of this row holds e_t
        const double et = __shfl(e, base + (t & (RL - 1)), 64);
        if (walked && t >= 0) pout = et / S;
    }

    if (live && l < G1) {
        int32_t o;
        if (invalid) o = -1;
        else if (l < n) o = tok;
        else if (l == n) o = t;
        else o = -1;
        p.tok_out[(int64_t)b * G1 + l] = o;
        const bool row_seen = !invalid && l <= n;
        if (p.aux_rmax) p.aux_rmax[(int64_t)b * G1 + l] = row_seen ? st_m : NAN;
        if (p.aux_rsum) p.aux_rsum[(int64_t)b * G1 + l] = row_seen && !GREEDY ? st_S : NAN;
        if (l < p.gamma) {
            if (p.aux_p) p.aux_p[(int64_t)b * p.gamma + l] = row_seen && !GREEDY ? st_P / st_S : NAN;
            if (p.aux_q) p.aux_q[(int64_t)b * p.gamma + l] = row_seen && !GREEDY ? st_Q : NAN;
        }
    }
    if (live && l == 0) {
        p.n_out[b] = invalid ? -1 : n;
        if (p.aux_resid) p.aux_resid[b] = invalid || GREEDY ? NAN : Z;
        if (p.aux_pout) p.aux_pout[b] = invalid || GREEDY ? NAN : pout;
    }
}

template <int DT, int PT>
bool launch_small_t(bool greedy, int tiny_lanes, int grid, const Params& p, hipStream_t s)
{
    if (tiny_lanes) {
        // k_tiny: rows of tiny_lanes lanes (8: eight sequences per wave, 16:
        // four); the rows of a sequence held in registers: 8 when gamma + 1 <= 8, else 16
        if (tiny_lanes == 8) {
            if (greedy) hipLaunchKernelGGL((k_tiny<DT, DT, true, 8, 8>), dim3(grid), dim3(kThreads), 0, s, p);
            else hipLaunchKernelGGL((k_tiny<DT, PT, false, 8, 8>), dim3(grid), dim3(kThreads), 0, s, p);
        } else if (p.gamma + 1 <= 8) {
            if (greedy) hipLaunchKernelGGL((k_tiny<DT, DT, true, 8, 16>), dim3(grid), dim3(kThreads), 0, s, p);
            else hipLaunchKernelGGL((k_tiny<DT, PT, false, 8, 16>), dim3(grid), dim3(kThreads), 0, s, p);
        } else {
            if (greedy) hipLaunchKernelGGL((k_tiny<DT, DT, true, kTinyV, 16>), dim3(grid), dim3(kThreads), 0, s, p);
            else hipLaunchKernelGGL((k_tiny<DT, PT, false, kTinyV, 16>), dim3(grid), dim3(kThreads), 0, s, p);
        }
        return hipGetLastError() == hipSuccess;
    }
    if (greedy) hipLaunchKernelGGL((k_small<DT, DT, true>), dim3(grid), dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((k_small<DT, PT, false>), dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError() == hipSuccess;
}

bool launch_small(int dt, int pt, bool greedy, int tiny_lanes, int grid, const Params& p, hipStream_t s)
{
    if (dt == SV_FP32 && (greedy || pt == SV_FP32)) return launch_small_t<SV_FP32, SV_FP32>(greedy, tiny_lanes, grid, p, s);
    if (dt == SV_FP32) return launch_small_t<SV_FP32, SV_BF16>(greedy, tiny_lanes, grid, p, s);
    if (greedy || pt == SV_FP32) return launch_small_t<SV_BF16, SV_FP32>(greedy, tiny_lanes, grid, p, s);
    return launch_small_t<SV_BF16, SV_BF16>(greedy, tiny_lanes, grid, p, s);
}

// ---------------------------------------------------------------- host dispatch

// lds1: dynamic LDS of the first launch, which only caps its workgroups per CU
template <int DT, int PT>
void launch_sample_t(int vmode, int grid1, unsigned lds1, int grid2, const Params& p, hipStream_t s,
                     hipEvent_t ev_mid, hipEvent_t ev_tele, bool* ok)
{
    switch (vmode) {
    case 2: hipLaunchKernelGGL((k_main_sample<DT, PT, 2>), dim3(grid1), dim3(kThreads), lds1, s, p); break;
    case 1: hipLaunchKernelGGL((k_main_sample<DT, PT, 1>), dim3(grid1), dim3(kThreads), lds1, s, p); break;
    default: hipLaunchKernelGGL((k_main_sample<DT, PT, 0>), dim3(grid1), dim3(kThreads), lds1, s, p); break;
    }
    if (hipGetLastError() != hipSuccess) { *ok = false; return; }
    if (ev_mid && hipEventRecord(ev_mid, s) != hipSuccess) { *ok = false; return; }
    if (p.tele) {
        const unsigned gridb = (unsigned)((size_t)p.B * p.gamma * p.nchb);
        if (vmode == 2) hipLaunchKernelGGL((k_beta<DT, PT, true>), dim3(gridb), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_beta<DT, PT, false>), dim3(gridb), dim3(kThreads), 0, s, p);
        hipLaunchKernelGGL(k_beta_merge, dim3((unsigned)p.gamma), dim3(kThreads), 0, s, p);
        if (hipGetLastError() != hipSuccess) { *ok = false; return; }
        if (ev_tele && hipEventRecord(ev_tele, s) != hipSuccess) { *ok = false; return; }
    }
    if (p.tele) {
        if (vmode == 2) hipLaunchKernelGGL((k_rest_sample<DT, PT, true>), dim3(grid2), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_rest_sample<DT, PT, false>), dim3(grid2), dim3(kThreads), 0, s, p);
    } else {
        if (vmode == 2) hipLaunchKernelGGL((k_finish_sample<DT, PT, true>), dim3(grid2), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_finish_sample<DT, PT, false>), dim3(grid2), dim3(kThreads), 0, s, p);
    }
    if (hipGetLastError() != hipSuccess) *ok = false;
}

bool launch_sample(int dt, int pt, int vmode, int grid1, unsigned lds1, int grid2, const Params& p, hipStream_t s,
                   hipEvent_t ev_mid, hipEvent_t ev_tele)
{
    bool ok = true;
    if (dt == SV_FP32 && pt == SV_FP32) launch_sample_t<SV_FP32, SV_FP32>(vmode, grid1, lds1, grid2, p, s, ev_mid, ev_tele, &ok);
    if (dt == SV_FP32 && pt == SV_BF16) launch_sample_t<SV_FP32, SV_BF16>(vmode, grid1, lds1, grid2, p, s, ev_mid, ev_tele, &ok);
    if (dt == SV_BF16 && pt == SV_FP32) launch_sample_t<SV_BF16, SV_FP32>(vmode, grid1, lds1, grid2, p, s, ev_mid, ev_tele, &ok);
    if (dt == SV_BF16 && pt == SV_BF16) launch_sample_t<SV_BF16, SV_BF16>(vmode, grid1, lds1, grid2, p, s, ev_mid, ev_tele, &ok);
    return ok;
}

template <int DT>
bool launch_greedy_t(bool vec, bool half_chunks, int grid1, unsigned lds1, int B, const Params& p, hipStream_t s,
                     hipEvent_t ev_mid)
{
    constexpr int EPT = DT == SV_BF16 ? kEptBf16 : kEptFp32;
    if (DT == SV_BF16 && half_chunks) {
        if (vec) hipLaunchKernelGGL((k_rows_greedy<DT, true, kEptFp32>), dim3(grid1), dim3(kThreads), lds1, s, p);
        else hipLaunchKernelGGL((k_rows_greedy<DT, false, kEptFp32>), dim3(grid1), dim3(kThreads), lds1, s, p);
    } else {
        if (vec) hipLaunchKernelGGL((k_rows_greedy<DT, true, EPT>), dim3(grid1), dim3(kThreads), lds1, s, p);
        else hipLaunchKernelGGL((k_rows_greedy<DT, false, EPT>), dim3(grid1), dim3(kThreads), lds1, s, p);
    }
    if (hipGetLastError() != hipSuccess) return false;
    if (ev_mid && hipEventRecord(ev_mid, s) != hipSuccess) return false;
    hipLaunchKernelGGL(k_draw_greedy, dim3(B), dim3(kThreads), 0, s, p);
    return hipGetLastError() == hipSuccess;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The launch geometry of one verify call: which kernels run on how many
// workgroups.  status is SV_ERR_TOO_LARGE when a grid would pass the limits
// (a grid's block count as int, nch1 within the 16 bits of a row counter,
// the batch within what a ready-list entry holds).
struct Plan {
    int nch1;          // row-stage chunks per row
    long long grid1;   // row-stage workgroups (G1 * B * nch1)
    long long gridh;   // first launch: the row stage, then B * nch2 draw helpers (sample, no telemetry)
    long long grid2;   // last launch: B (greedy, or with helpers) or B * nch2 (telemetry)
    long long gridb;   // telemetry sweep: B * gamma * nchb
    bool small;        // V <= 512 without telemetry: one launch of k_small or k_tiny
    bool tiny;         //   k_tiny: V <= 16 and gamma < 16
    int tiny_lanes;    //   its lanes per sequence: 8 when V <= 8 and gamma < 8, else 16
    int seqs_per_wg;   //   sequences per workgroup of the one launch
    long long grid_small;
    bool helpers;
    bool half_chunks;  //   greedy, bf16 rows: kChunkFp32-entry row chunks (a small batch)
    bool fine;         //   one helper per sub-chunk (at most kFineHelpers of them), else one per draw chunk
    int status;
};

Plan make_plan(int batch, int gamma, int vocab, int logits_dtype, bool greedy, bool tele)
{
    const Layout L = make_layout(batch, gamma, vocab);
    Plan q{};
    const int chunk1 = logits_dtype == SV_BF16 ? kChunkBf16 : kChunkFp32;
    q.nch1 = (vocab + chunk1 - 1) / chunk1;
    // greedy calls on bf16 rows whose positions hold few row blocks take
    // half-size chunks: shorter blocks move the decisions along sooner
    q.half_chunks = greedy && logits_dtype == SV_BF16 && (long long)batch * q.nch1 <= kHalfChunkBlocks;
    if (q.half_chunks) q.nch1 = (vocab + kChunkFp32 - 1) / kChunkFp32;
    q.grid1 = (long long)(gamma + 1) * batch * q.nch1;
    q.helpers = !greedy && !tele;
    q.fine = q.helpers && (long long)batch * L.nsub <= kFineHelpers;
    q.gridh = q.helpers ? q.grid1 + (long long)batch * (q.fine ? L.nsub : L.nch2) : q.grid1;
    q.grid2 = greedy || q.helpers ? (long long)batch : (long long)batch * L.nch2;
    q.gridb = tele ? (long long)batch * gamma * L.nchb : 0;
    q.small = vocab <= kSmallV && !tele;
    q.tiny = q.small && vocab <= kTinyV && gamma < 16;
    q.tiny_lanes = vocab <= 8 && gamma + 1 <= 8 ? 8 : 16;
    q.seqs_per_wg = q.tiny ? (64 / q.tiny_lanes) * kWaves : kWaves;
    q.grid_small = ((long long)batch + q.seqs_per_wg - 1) / q.seqs_per_wg;
    q.status = SV_OK;
    if (q.nch1 > 0xffff || q.gridh > INT_MAX || q.grid2 > INT_MAX || q.gridb > INT_MAX) q.status = SV_ERR_TOO_LARGE;
    if (!greedy && batch > kMaxListed) q.status = SV_ERR_TOO_LARGE;
    return q;
}

// Row blocks resident per CU in the first launch.  Rows past a sequence's
// first rejection are skipped only once that rejection is known, and position
// k's blocks are dispatched after those of every earlier position; with the
// batch resident several positions deep, the later positions stream rows that
// the earlier ones are about to make unneeded.  A few positions of row blocks
// at a time (B * nch1 blocks a position) keep the chip fed while the
// decisions stay ahead: ceil(depth * blocks / CUs), between 3 and 8 (8: no
// cap, the kernel's own limit at <= 64 VGPRs).  The depth, in half positions:
// 3 in sample mode, 4 in greedy mode, whose rejections land sooner (any chunk
// with an entry above the draft token's decides its position).
constexpr int kMinRowWgsPerCu = 3, kMaxRowWgsPerCu = 8;
constexpr int kSampleHalfPositions = 3, kGreedyHalfPositions = 4;
constexpr int kStaticLdsMargin = 256;  // above the first launch's static LDS (< 200 bytes)

inline int row_wgs_per_cu(long long blocks_per_position, int n_cu, int half_positions)
{
    if (n_cu <= 0) return kMaxRowWgsPerCu;
    const long long n = (half_positions * blocks_per_position + 2LL * n_cu - 1) / (2LL * n_cu);
    return (int)(n < kMinRowWgsPerCu ? kMinRowWgsPerCu : n > kMaxRowWgsPerCu ? kMaxRowWgsPerCu : n);
}

// Dynamic LDS that holds a workgroup to `wgs` per CU (0: no cap): each takes
// lds_cu / (wgs + 1/2) bytes, static LDS included, so `wgs` of them fit and
// one more does not; the slack, lds_cu / (2 wgs + 1), covers the allocation
// granule.
inline unsigned cap_lds_bytes(int wgs, int lds_cu, int lds_block_max)
{
    if (wgs >= kMaxRowWgsPerCu || wgs < 1 || lds_cu <= 0) return 0u;
    const long long dyn = 2LL * lds_cu / (2 * wgs + 1) - kStaticLdsMargin;
    return dyn > 0 && dyn + kStaticLdsMargin <= lds_block_max ? (unsigned)dyn : 0u;
}

// The checks of every verify entry point that need no workspace and no HIP
// call; SV_OK or the status to return.
int check_args(int batch, int gamma, int vocab, const void* target_logits, int logits_dtype,
               const void* draft_probs, int probs_dtype, const int32_t* draft_tokens, const float* uniforms,
               float temperature, float lenience, int mode, const int32_t* n_accepted, const int32_t* out_tokens)
{
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
        if (!(lenience >= 0.0f && lenience <= 1.0f)) return SV_ERR_LENIENCE;
    }
    const size_t lsz = logits_dtype == SV_BF16 ? 2 : 4;
    const size_t psz = probs_dtype == SV_BF16 ? 2 : 4;
    if (!aligned(target_logits, lsz) || !aligned(draft_tokens, 4) || !aligned(n_accepted, 4) ||
        !aligned(out_tokens, 4))
        return SV_ERR_ALIGNMENT;
    if (!greedy && (!aligned(draft_probs, psz) || !aligned(uniforms, 4))) return SV_ERR_ALIGNMENT;
    return SV_OK;
}

}  // namespace

// The workspace of spec_verify_noalloc: one file-scope device array per GPU
// the library runs on, held until the process ends.  Host code never passes
// the array's name to a kernel or a copy (on the host it is only a
// stand-in): it uses the device address that hipGetSymbolAddress returns,
// fetched once per device with that device current.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's CU count and LDS sizes, asked once per device; zeros
// when they cannot be had (the first launch then runs uncapped).
struct DevProps {
    int n_cu, lds_cu, lds_block;
};
std::mutex g_props_mu;
DevProps g_props[kMaxDevices] = {};

DevProps dev_props()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DevProps{0, 0, 0};
    std::lock_guard<std::mutex> lock(g_props_mu);
    DevProps& d = g_props[dev];
    if (d.n_cu == 0) {
        DevProps q{0, 0, 0};
        if (hipDeviceGetAttribute(&q.n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&q.lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            hipDeviceGetAttribute(&q.lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return DevProps{0, 0, 0};
        d = q;
    }
    return d;
}

// The current device's scratch address, fetched and zero-filled (with a
// kernel, on `s`) on the first call on that device; nullptr on failure.
void* scratch_for_current_device(hipStream_t s)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    // (a workspace must be zero before its first use)
    constexpr size_t n16 = SV_NOALLOC_SCRATCH_BYTES / 16;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                       static_cast<uint4*>(ptr), n16, static_cast<unsigned char*>(ptr), (size_t)0);
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
    return ptr;
}

}  // namespace

extern "C" {

size_t sv_extras_bytes(void) { return sizeof(sv_extras_t); }

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
    return spec_verify_lenient(batch, gamma, vocab, target_logits, logits_dtype, draft_probs, probs_dtype,
                               draft_tokens, uniforms, temperature, 1.0f, mode, n_accepted, out_tokens,
                               workspace, workspace_bytes, extras, stream);
}

int spec_verify_lenient(int batch, int gamma, int vocab,
                        const void* target_logits, int logits_dtype,
                        const void* draft_probs, int probs_dtype,
                        const int32_t* draft_tokens, const float* uniforms,
                        float temperature, float lenience, int mode,
                        int32_t* n_accepted, int32_t* out_tokens,
                        void* workspace, size_t workspace_bytes,
                        const sv_extras_t* extras, void* stream)
{
    // ---- argument validation (no HIP call before this block passes)
    const int bad = check_args(batch, gamma, vocab, target_logits, logits_dtype, draft_probs, probs_dtype,
                               draft_tokens, uniforms, temperature, lenience, mode, n_accepted, out_tokens);
    if (bad != SV_OK) return bad;
    const bool greedy = mode == SV_GREEDY;
    const size_t lsz = logits_dtype == SV_BF16 ? 2 : 4;
    const Layout L = make_layout(batch, gamma, vocab);
    if (!workspace || workspace_bytes < L.total) return SV_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SV_ERR_ALIGNMENT;

    const bool tele = !greedy && extras && (extras->beta || extras->alpha);
    // sample mode without telemetry: draw helpers follow the row blocks of
    // the first launch, and the last launch is one workgroup per sequence
    const Plan q = make_plan(batch, gamma, vocab, logits_dtype, greedy, tele);
    if (q.status != SV_OK) return q.status;
    const int nch1 = q.nch1;
    // vector loads need 16-byte aligned rows: in the row stage of the logits,
    // in the draw of the logits and the draft probabilities (8 elements)
    const bool vec = aligned(target_logits, 16) && ((size_t)vocab * lsz) % 16 == 0;
    const bool vec2 = vec && vocab % 8 == 0 && (greedy || aligned(draft_probs, 16));
    const int vmode = vec2 ? 2 : vec ? 1 : 0;

    char* ws = static_cast<char*>(workspace);
    hipStream_t s = (hipStream_t)stream;

    // log2(e)/T as c_hi + c_lo with c_hi <= log2(e)/T, so c_lo > 0 and
    // -inf logits stay -inf through both fused multiply-adds
    const double cd = greedy ? 0.0 : kLog2e / (double)temperature;
    float c_hi = (float)cd;
    if ((double)c_hi >= cd) c_hi = std::nextafter(c_hi, 0.0f);
    const float c_lo = (float)(cd - (double)c_hi);

    Params p;
    p.logits = target_logits;
    p.probs = greedy ? nullptr : draft_probs;
    p.tokens = draft_tokens;
    p.uniforms = uniforms;
    p.ctl = reinterpret_cast<SeqCtl*>(ws + L.ctl_off);
    p.cnt1 = reinterpret_cast<uint64_t*>(ws + L.cnt1_off);
    p.part1 = reinterpret_cast<uint64_t*>(ws + L.part1_off);
    p.stats = reinterpret_cast<RowStat*>(ws + L.stats_off);
    p.sub = reinterpret_cast<SubSum*>(ws + L.sub_off);
    p.ready = reinterpret_cast<uint32_t*>(ws + L.ready_off);
    p.ready_cnt = reinterpret_cast<uint32_t*>(ws + L.rcnt_off);
    p.n_out = n_accepted;
    p.tok_out = out_tokens;
    p.aux_p = extras ? extras->p_tok : nullptr;
    p.aux_q = extras ? extras->q_tok : nullptr;
    p.aux_resid = extras ? extras->resid_mass : nullptr;
    p.aux_pout = extras ? extras->p_out : nullptr;
    p.aux_rmax = extras ? extras->row_max : nullptr;
    p.aux_rsum = extras ? extras->row_sum : nullptr;
    p.aux_beta = tele ? extras->beta : nullptr;
    p.aux_alpha = tele ? extras->alpha : nullptr;
    p.bpart = reinterpret_cast<double*>(ws + L.bpart_off);
    p.tele = tele ? 1 : 0;
    p.nchb = L.nchb;
    p.B = batch;
    p.gamma = gamma;
    p.V = vocab;
    p.nch1 = nch1;
    p.nch2 = L.nch2;
    p.nsub = L.nsub;
    p.fine = q.fine ? 1 : 0;
    p.probs_dtype = probs_dtype;
    p.zero = 0u;
    p.c_hi = c_hi;
    p.c_lo = c_lo;
    p.cd = cd;
    p.ex = kExp2Coef;
    p.len = greedy ? 1.0 : (double)lenience;
    p.rows_grid = (int)q.grid1;
    p.help_polls = extras && extras->help_polls > 0 ? extras->help_polls : kHelpPolls;
    p.polls_slot = extras && extras->wait_polls > 0 ? extras->wait_polls : kSlotPolls;
    p.drop_slot = extras && extras->withhold_partial > 0 ? extras->withhold_partial - 1 : -1;
    p.err_count = extras ? extras->error_count : nullptr;

    hipEvent_t ev_mid = extras ? (hipEvent_t)extras->ev_mid : nullptr;
    if (extras && extras->ev_begin && hipEventRecord((hipEvent_t)extras->ev_begin, s) != hipSuccess)
        return SV_ERR_LAUNCH;
    bool ok;
    if (q.small) {
        // one launch, one wave per sequence (the workspace is not touched)
        ok = launch_small(logits_dtype, probs_dtype, greedy, q.tiny ? q.tiny_lanes : 0, (int)q.grid_small, p, s);
        if (ok && ev_mid && hipEventRecord(ev_mid, s) != hipSuccess) ok = false;
    } else {
        // the first launch's cap on resident row blocks, only where rows can
        // be skipped (the telemetry streams every row)
        unsigned lds1 = 0;
        if (greedy || q.helpers) {
            const DevProps dp = dev_props();
            const int depth = greedy ? kGreedyHalfPositions : kSampleHalfPositions;
            lds1 = cap_lds_bytes(row_wgs_per_cu((long long)batch * nch1, dp.n_cu, depth), dp.lds_cu, dp.lds_block);
        }
        if (greedy)
            ok = logits_dtype == SV_BF16
                     ? launch_greedy_t<SV_BF16>(vec, q.half_chunks, (int)q.grid1, lds1, batch, p, s, ev_mid)
                     : launch_greedy_t<SV_FP32>(vec, false, (int)q.grid1, lds1, batch, p, s, ev_mid);
        else
            ok = launch_sample(logits_dtype, probs_dtype, vmode, (int)q.gridh, lds1, (int)q.grid2, p, s, ev_mid,
                               extras ? (hipEvent_t)extras->ev_tele : nullptr);
    }
    if (!ok) return SV_ERR_LAUNCH;
    if (extras && extras->ev_end && hipEventRecord((hipEvent_t)extras->ev_end, s) != hipSuccess)
        return SV_ERR_LAUNCH;
    return SV_OK;
}

int spec_verify_noalloc(int batch, int gamma, int vocab,
                        const void* target_logits, int logits_dtype,
                        const void* draft_probs, int probs_dtype,
                        const int32_t* draft_tokens, const float* uniforms,
                        float temperature, float lenience, int mode,
                        int32_t* n_accepted, int32_t* out_tokens,
                        const sv_extras_t* extras, void* stream)
{
    const int bad = check_args(batch, gamma, vocab, target_logits, logits_dtype, draft_probs, probs_dtype,
                               draft_tokens, uniforms, temperature, lenience, mode, n_accepted, out_tokens);
    if (bad != SV_OK) return bad;
    if (sv_workspace_bytes(batch, gamma, vocab) > SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_SCRATCH;
    void* ws = scratch_for_current_device((hipStream_t)stream);
    if (!ws) return SV_ERR_LAUNCH;
    return spec_verify_lenient(batch, gamma, vocab, target_logits, logits_dtype, draft_probs, probs_dtype,
                               draft_tokens, uniforms, temperature, lenience, mode, n_accepted, out_tokens,
                               ws, SV_NOALLOC_SCRATCH_BYTES, extras, stream);
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
    case SV_ERR_LENIENCE: return "lenience must be in [0, 1] in sample mode";
    case SV_ERR_STANDARDIZE: return "standardisation needs SV_TOPK with k >= 1 or SV_TOPP with 0 < top_p <= 1";
    case SV_ERR_SCRATCH: return "spec_verify_noalloc: the problem needs more workspace than its static scratch array (SV_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

}  // extern "C"
