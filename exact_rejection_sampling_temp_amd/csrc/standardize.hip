// standardize.hip -- top-k and nucleus standardisation of rows of logits on
// MI355X (gfx950).
//
// "Fast Inference from Transformers via Speculative Decoding" (paper summary
// page), "Standardized Sampling": every sampling method is plain sampling
// from an adjusted distribution -- top-k keeps the k largest probabilities,
// nucleus keeps the shortest run of the largest probabilities whose sum
// reaches top_p -- and the verify step compares those adjusted
// distributions.  The output here is the row of logits with every dropped
// entry set to -inf, so the temperature softmax of the output is exactly the
// renormalised kept set, and spec_verify runs on it unchanged.
//
// One workgroup per row.  Entries are compared through order-preserving
// integer keys (larger value <=> larger key, -0 folded onto +0).  The
// selection finds the final key k* (the smallest kept value) and how many of
// the entries equal to it are kept; ties are kept first in index order, so
// top-k keeps exactly min(k, V) entries.
//
// bf16 rows (k_standardize_b16): a bf16 value has only 2^16 patterns, so one
// pass over the row counts every key in a 65 536-entry histogram of 16-bit
// counters held in LDS (128 KiB; two counters per 32-bit word, updated with
// ds_add_u32 of 1 or 1 << 16).  A workgroup scan over the keys from the top
// then gives k* exactly: by count for top-k, and for the nucleus by mass,
// where a key's mass is its count times exp((z - max)/T), one fp64
// exponential per distinct value instead of one per entry.  The row maximum
// is the highest key present.  If any value occurs 65 536 times or more
// (which the total count reveals) the row falls back to the radix select
// below.
//
// fp32 rows (k_standardize), and the fallback: an MSB-first radix select
// (12-, 12- then 8-bit digits; 12 then 4 for bf16): a pass over the row
// builds the digit's histogram in LDS (counts, and for the nucleus fp64
// masses), a scan over the bins from the top finds the bin where the count
// (mass) crosses k (top_p times the row's mass), and the next pass refines
// inside that bin.
//
// Every pass walks the row the same way, each wave over a contiguous run of
// it, with kUnroll groups of 8 entries per lane in flight.  The output pass
// needs, for each wave, the number of entries equal to k* in the runs before
// its own: a wave whose run lies wholly before the last kept tie or wholly
// after it keeps entries by a key threshold (for bf16 two entries per 32-bit
// operation), and only a wave whose run holds the last kept tie ranks its
// ties in index order.  The output is written with 128-bit nontemporal
// stores where the row allows.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "spec_verify.h"

namespace {

#ifndef SV_STD_TOPK_THREADS
#define SV_STD_TOPK_THREADS 512
#endif
#ifndef SV_STD_NUC_THREADS
#define SV_STD_NUC_THREADS 512
#endif
#ifndef SV_STD_UNROLL
#define SV_STD_UNROLL 4
#endif
// radix-select workgroups (fp32 rows): 512 threads, two rows per CU
template <bool NUCLEUS>
struct StdShape {
    static constexpr int kSThreads = NUCLEUS ? SV_STD_NUC_THREADS : SV_STD_TOPK_THREADS;
    static constexpr int kSWaves = kSThreads / 64;
};
constexpr int kMaxWaves = 16;
constexpr int kBins = 4096;  // 12-bit digits
// groups of 8 bf16 entries per thread per pass iteration (loads in flight);
// fp32 rows take half as many groups (the same bytes), the scalar-load path 2
constexpr int kUnroll = SV_STD_UNROLL;
template <int DT, bool VEC>
constexpr int unroll_of() { return VEC ? (DT == SV_BF16 ? kUnroll : kUnroll / 2) : 2; }

// bf16 workgroups: 1024 threads, one row per CU (the histogram takes 128 KiB)
constexpr int kHThreads = 1024;
constexpr int kHWaves = kHThreads / 64;
constexpr int kHWords = 32768;                      // 65 536 16-bit counters
constexpr uint32_t kTieCap = 1024;                  // listed ties per wave (64 KiB of the histogram's space)

struct StdParams {
    const void* in;
    void* out;
    int V, method, k;
    double top_p;
    double cd;  // log2(e)/T
};

// Order-preserving keys: a value with sign bit s and magnitude bits a maps
// to H + a when s = 0 and H - a when s = 1 (H = 2^15 for bf16, 2^31 for
// fp32), so -0 and +0 share the key H and larger values have larger keys.
template <int DT>
__device__ __forceinline__ uint32_t key_of(uint32_t bits)
{
    constexpr uint32_t H = DT == SV_BF16 ? 0x8000u : 0x80000000u;
    const uint32_t mag = bits & (H - 1u);
    return (bits & H) ? H - mag : H + mag;
}
template <int DT>
__device__ __forceinline__ uint32_t bits_of_key(uint32_t key)
{
    constexpr uint32_t H = DT == SV_BF16 ? 0x8000u : 0x80000000u;
    return key >= H ? key - H : H | (H - key);
}
template <int DT>
__device__ __forceinline__ float value_of_bits(uint32_t bits)
{
    if constexpr (DT == SV_BF16) return __uint_as_float(bits << 16);
    else return __uint_as_float(bits);
}
template <int DT>
__device__ __forceinline__ float value_of_key(uint32_t key) { return value_of_bits<DT>(bits_of_key<DT>(key)); }

// The keys of the two bf16 patterns packed in a 32-bit word, packed the same
// way (key_of<SV_BF16> of each half, with 16-bit vector operations).
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t keys2(uint32_t w)
{
    const s16x2 x = __builtin_bit_cast(s16x2, w);
    const s16x2 s = x >> (s16x2)15;           // 0 or -1 per half
    const s16x2 mag = x & (s16x2)0x7fff;
    const s16x2 sm = (mag ^ s) - s;           // -a for negative values, a otherwise
    return __builtin_bit_cast(uint32_t, sm) ^ 0x80008000u;
}
// The two packed bf16 patterns of w where their key (packed in k2) is >=
// kcut (kcut2 holds kcut in both halves), -inf where it is below.
__device__ __forceinline__ uint32_t keep2(uint32_t w, uint32_t k2, uint32_t kcut2)
{
    const u16x2 k = __builtin_bit_cast(u16x2, k2);
    const u16x2 below = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, kcut2), k);  // 0 iff kept
    const u16x2 drop = (u16x2)0 - __builtin_elementwise_min(below, (u16x2)1);              // 0xffff iff dropped
    const uint32_t m = __builtin_bit_cast(uint32_t, drop);
    return (w & ~m) | (0xff80ff80u & m);
}

// 8 consecutive raw elements (bit patterns) starting at index base, kept as
// loaded: bf16 packs two patterns per word in a, fp32 uses a and b.  Entries
// at or past V hold whatever the clamped loads return; callers test
// base + e < V.  VEC: 16-byte aligned rows (full groups load 128 bits).
struct G8 {
    uint4 a, b;
};
template <int DT, bool VEC>
__device__ __forceinline__ G8 load_g8(const void* row, int base, int V)
{
    G8 r;
    r.b = make_uint4(0u, 0u, 0u, 0u);
    if (VEC && base + 8 <= V) {
        if constexpr (DT == SV_BF16) {
            r.a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + base);
        } else {
            r.a = *reinterpret_cast<const uint4*>(static_cast<const float*>(row) + base);
            r.b = *reinterpret_cast<const uint4*>(static_cast<const float*>(row) + base + 4);
        }
        return r;
    }
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int i = min(base + e, V - 1);
        if constexpr (DT == SV_BF16) v[e] = static_cast<const uint16_t*>(row)[i];
        else v[e] = static_cast<const uint32_t*>(row)[i];
    }
    if constexpr (DT == SV_BF16) {
        r.a = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
    } else {
        r.a = make_uint4(v[0], v[1], v[2], v[3]);
        r.b = make_uint4(v[4], v[5], v[6], v[7]);
    }
    return r;
}
template <int DT>
__device__ __forceinline__ uint32_t bits_of(const G8& g, int e)
{
    if constexpr (DT == SV_BF16) {
        const uint32_t w = e < 2 ? g.a.x : e < 4 ? g.a.y : e < 6 ? g.a.z : g.a.w;
        return (e & 1) ? (w >> 16) : (w & 0xffffu);
    } else {
        return e == 0 ? g.a.x : e == 1 ? g.a.y : e == 2 ? g.a.z : e == 3 ? g.a.w
             : e == 4 ? g.b.x : e == 5 ? g.b.y : e == 6 ? g.b.z : g.b.w;
    }
}
__device__ __forceinline__ uint32_t word_of(const uint4& a, int i) { return i == 0 ? a.x : i == 1 ? a.y : i == 2 ? a.z : a.w; }

// 16-byte store of the output, nontemporal: the output is not read again
// here, and streaming it past the caches leaves them to the input rows
// (measured 1-3 % faster on the c4 rows)
__device__ __forceinline__ void store16(void* p, uint4 v)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// 2^a in fp64: round to the nearest integer n, a degree-9 polynomial for
// 2^f on f in [-1/2, 1/2] (Taylor coefficients (ln 2)^i / i! of e^(f ln 2);
// relative error below 7e-12, far inside the 1e-9 window the nucleus
// boundary is judged in), then ldexp.  a <= 0 here (entries relative to the
// row maximum).
__device__ __forceinline__ double exp2_fast(double a)
{
    constexpr double kMagic = 6755399441055744.0;  // 1.5 * 2^52
    a = fmax(a, -1100.0);
    const double t = a + kMagic;
    const double f = a - (t - kMagic);
    const int n = __double2loint(t);
    constexpr double c[10] = {1.0, 0.6931471805599453, 0.2402265069591007, 0.05550410866482158,
                              0.009618129107628477, 0.0013333558146428443, 0.00015403530393381606,
                              1.525273380405984e-05, 1.3215486790144307e-06, 1.0178086009239699e-07};
    double p = c[9];
#pragma unroll
    for (int i = 8; i >= 0; --i) p = fma(f, p, c[i]);
    return ldexp(p, n);
}

template <typename T>
__device__ __forceinline__ T wave_incl_scan_t(T v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const T t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Sum of v over each 32-lane half of the wave, in every lane of the half:
// DPP within the 16-lane rows (quad swaps, half-row and row mirrors), then
// one exchange between the two rows of the half.
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xf, 0xf, false);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double half_wave_sum(double v)
{
    v += dpp_d<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_d<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_d<0x141>(v);  // row_half_mirror
    v += dpp_d<0x140>(v);  // row_mirror
    return v + __shfl_xor(v, 16, 64);
}

// Exclusive scan over the workgroup in thread order; *total gets the sum.
template <typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* sm, T* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nw = (int)(blockDim.x >> 6);
    const T incl = wave_incl_scan_t(v);
    if (lane == 63) sm[w] = incl;
    __syncthreads();
    T before = T(0), all = T(0);
#pragma unroll
    for (int i = 0; i < kMaxWaves; ++i) {
        if (i >= nw) break;
        const T s = sm[i];
        if (i < w) before += s;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

// block_excl_scan of a count and a mass together (one pair of barriers).
__device__ __forceinline__ void block_excl_scan2(uint32_t c, double m, uint32_t* smu, double* smd, uint32_t* c_before,
                                                 double* m_before, uint32_t* c_total, double* m_total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nw = (int)(blockDim.x >> 6);
    const uint32_t ci = wave_incl_scan_t(c);
    const double mi = wave_incl_scan_t(m);
    if (lane == 63) { smu[w] = ci; smd[w] = mi; }
    __syncthreads();
    uint32_t cb = 0, ca = 0;
    double mb = 0.0, ma = 0.0;
#pragma unroll
    for (int i = 0; i < kMaxWaves; ++i) {
        if (i >= nw) break;
        const uint32_t sc = smu[i];
        const double sd = smd[i];
        if (i < w) { cb += sc; mb += sd; }
        ca += sc;
        ma += sd;
    }
    __syncthreads();
    *c_before = cb + ci - c;
    *m_before = mb + mi - m;
    *c_total = ca;
    *m_total = ma;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* sm)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t r = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r = max(r, sm[i]);
    __syncthreads();
    return r;
}

// Small shared state of one row.
struct StdSmall {
    uint32_t u[kMaxWaves];
    double d[kMaxWaves];
    uint32_t tw[kMaxWaves];  // entries equal to the final key in each wave's run
    uint32_t bin, above_cnt, kstar, need, found, partial;
    double above_mass;
    uint32_t tcross, cb;  // the thread whose keys hold the crossing, and the count above them
    double mb;            // the mass above them
    uint32_t kmax[kMaxWaves];  // bf16 kernel: each wave's largest key (the row maximum)
};

// The selection's result for one row.
struct Sel {
    bool keep_all;
    uint32_t kstar;  // the final key
    uint32_t need;   // entries equal to kstar that are kept, first in index order
};

// A wave's contiguous run of 8-entry groups [g_begin, g_end): a multiple of
// 64 groups long; lane l takes groups g_begin + 64 j + l, so a wave's
// entries are visited in index order by (j, lane, entry).
struct Run {
    int g_begin, g_end;
    __device__ Run(int ngroups, int nwaves)
    {
        const int seg = ((ngroups + nwaves - 1) / nwaves + 63) & ~63;
        g_begin = min(ngroups, (int)(threadIdx.x >> 6) * seg);
        g_end = min(ngroups, g_begin + seg);
    }
};

// ------------------------------------------------------------ radix select

// Radix select of one row (see the file comment).  h_cnt: kBins counters;
// h_mass: kBins doubles (nucleus); h_tot: the last digit's totals.  Fills
// sm.tw with each wave's count of entries equal to the final key.
template <int DT, bool VEC, bool NUCLEUS>
__device__ __forceinline__ Sel radix_select(const StdParams& sp, const void* row, const Run& run, uint32_t* h_cnt, double* h_mass,
                            uint32_t* h_tot, StdSmall& sm)
{
    const int nthreads = (int)blockDim.x;
    const int nw = nthreads >> 6;
    const int bins_per_thread = kBins / nthreads;
    constexpr int KB = DT == SV_BF16 ? 16 : 32;
    constexpr int NPASS = DT == SV_BF16 ? 2 : 3;
    constexpr int kShift[3] = {KB - 12, DT == SV_BF16 ? 0 : 8, 0};
    constexpr int kDigit[3] = {12, DT == SV_BF16 ? 4 : 12, 8};
    constexpr int kLastBins = 1 << kDigit[NPASS - 1];  // bins of the last digit
    static_assert(kMaxWaves * kLastBins <= kBins, "per-wave last-digit histograms share the bin array");
    constexpr int U = unroll_of<DT, VEC>();
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int V = sp.V;
    const int g_begin = run.g_begin, g_end = run.g_end;

    // the row maximum (nucleus masses are taken relative to it)
    double m = 0.0;
    if (NUCLEUS) {
        uint32_t mk = 0;
        for (int j0 = g_begin; j0 < g_end; j0 += U * 64) {  // uniform trip count
            G8 gu[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = j0 + u * 64 + lane;
                gu[u] = g < g_end ? load_g8<DT, VEC>(row, g * 8, V) : G8{};
            }
#pragma unroll
            for (int ue = 0; ue < U * 8; ++ue) {
                const int g = j0 + (ue >> 3) * 64 + lane;
                if (g < g_end && g * 8 + (ue & 7) < V) mk = max(mk, key_of<DT>(bits_of<DT>(gu[ue >> 3], ue & 7)));
            }
        }
        m = (double)value_of_key<DT>(block_max_u32(mk, sm.u));
    }

    Sel sel{false, 0u, 0u};
    uint32_t prefix = 0;
    uint32_t rem_cnt = (uint32_t)min(sp.k, V);
    double rem_mass = 0.0;
    for (int ps = 0; ps < NPASS; ++ps) {
        const int shift = kShift[ps], dbits = kDigit[ps];
        const uint32_t dmask = (1u << dbits) - 1u;
        const bool last = ps == NPASS - 1;
        // the last digit's counts go to per-wave copies (wave w's at
        // w * kLastBins), from which each wave's ties follow
        const int cbase = last ? wv * kLastBins : 0;
        for (int i = tid; i < kBins; i += nthreads) {
            h_cnt[i] = 0u;
            if (NUCLEUS) h_mass[i] = 0.0;
        }
        __syncthreads();
        for (int j0 = g_begin; j0 < g_end; j0 += U * 64) {  // uniform trip count
            G8 gu[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {  // every load of the iteration in flight at once
                const int g = j0 + u * 64 + lane;
                gu[u] = g < g_end ? load_g8<DT, VEC>(row, g * 8, V) : G8{};
            }
#pragma unroll
            for (int ue = 0; ue < U * 8; ++ue) {
                const int e = ue & 7;
                const int g = j0 + (ue >> 3) * 64 + lane;
                const uint32_t bits = bits_of<DT>(gu[ue >> 3], e);
                const uint32_t key = key_of<DT>(bits);
                const uint32_t hi = shift + dbits >= 32 ? 0u : (key >> (shift + dbits));
                if (g >= g_end || g * 8 + e >= V || hi != prefix) continue;
                const uint32_t bin = (key >> shift) & dmask;
                atomicAdd(&h_cnt[cbase + bin], 1u);
                if (NUCLEUS) {
                    const float z = value_of_bits<DT>(bits);
                    if (z > -INFINITY) atomicAdd(&h_mass[bin], exp2_fast(((double)z - m) * sp.cd));
                }
            }
        }
        __syncthreads();
        if (last) {
            for (int b = tid; b < kLastBins; b += nthreads) {
                uint32_t s = 0;
                for (int w = 0; w < nw; ++w) s += h_cnt[w * kLastBins + b];
                h_tot[b] = s;
            }
            __syncthreads();
        }
        auto count_of = [&](int b) -> uint32_t { return last ? (b < kLastBins ? h_tot[b] : 0u) : h_cnt[b]; };
        // bins from the top: thread t takes bins 4095 - bpt t - i, i < bpt
        uint32_t c_loc = 0;
        double m_loc = 0.0;
        for (int i = 0; i < bins_per_thread; ++i) {
            const int b = kBins - 1 - (bins_per_thread * tid + i);
            c_loc += count_of(b);
            if (NUCLEUS) m_loc += h_mass[b];
        }
        uint32_t c_tot;
        double m_tot = 0.0;
        uint32_t c_before = block_excl_scan<uint32_t>(c_loc, sm.u, &c_tot);
        double m_before = NUCLEUS ? block_excl_scan<double>(m_loc, sm.d, &m_tot) : 0.0;
        if (ps == 0 && NUCLEUS) rem_mass = sp.top_p * m_tot;  // the row's mass, summed once
        if (tid == 0) sm.bin = 0xffffffffu;
        __syncthreads();
        for (int i = 0; i < bins_per_thread; ++i) {
            const int b = kBins - 1 - (bins_per_thread * tid + i);
            const uint32_t hc = count_of(b);
            const double hm = NUCLEUS ? h_mass[b] : 0.0;
            const bool cross = NUCLEUS ? (hc > 0 && m_before < rem_mass && rem_mass <= m_before + hm)
                                       : (c_before < rem_cnt && rem_cnt <= c_before + hc);
            if (cross) {
                sm.bin = (uint32_t)b;
                sm.above_cnt = c_before;
                sm.above_mass = m_before;
            }
            c_before += hc;
            m_before += hm;
        }
        __syncthreads();
        const uint32_t bin = sm.bin;
        if (bin == 0xffffffffu) {
            sel.keep_all = true;  // the running mass never reaches top_p (rounding): keep every entry
            return sel;
        }
        prefix = (prefix << dbits) | bin;
        rem_cnt -= sm.above_cnt;
        rem_mass -= sm.above_mass;
        if (last && tid < nw) sm.tw[tid] = h_cnt[tid * kLastBins + bin];
        __syncthreads();
    }
    sel.kstar = prefix;
    sel.need = rem_cnt;
    if (NUCLEUS) {
        const double wt = exp2_fast(((double)value_of_key<DT>(prefix) - m) * sp.cd);
        const double n = ceil(rem_mass / wt);
        sel.need = n < 1.0 ? 1u : (n > 4294967295.0 ? 0xffffffffu : (uint32_t)n);
    }
    return sel;
}

// ------------------------------------------------------------ output pass

// Writes the row: entries above the final key as they are, ties kept by
// index order up to sel.need, the rest -inf.  tb / tw: entries equal to the
// final key before this wave's run / in it.  COLLECT (tw unknown): every tie
// is kept, and the wave's ties are numbered in index order, the index of
// the first cap of them stored in list; returns how many there are.
template <int DT, bool VEC, bool COLLECT = false>
__device__ __forceinline__ uint32_t write_row(const StdParams& sp, const void* row, void* orow, const Run& run, const Sel& sel,
                              uint32_t tb, uint32_t tw, uint32_t* list = nullptr, uint32_t cap = 0)
{
    constexpr int U = unroll_of<DT, VEC>();
    constexpr uint32_t kKeyMax = DT == SV_BF16 ? 0xffffu : 0xffffffffu;
    constexpr uint32_t kNegInf = DT == SV_BF16 ? 0xff80u : 0xff800000u;
    const int lane = (int)threadIdx.x & 63;
    const int V = sp.V;
    const int g_begin = run.g_begin, g_end = run.g_end;
    // a key threshold for the whole run, unless the run holds the last kept tie
    bool ranked = false;
    uint32_t kcut = 0;
    if (COLLECT) {
        kcut = sel.kstar;
    } else if (!sel.keep_all) {
        if (tb + tw <= sel.need) kcut = sel.kstar;                              // every tie of the run kept
        else if (tb >= sel.need && sel.kstar < kKeyMax) kcut = sel.kstar + 1u;  // none kept
        else ranked = true;
    }
    uint32_t running = COLLECT ? 0u : tb;
    const uint32_t ks2 = sel.kstar | (sel.kstar << 16);
    for (int j0 = g_begin; j0 < g_end; j0 += U * 64) {  // uniform trip count
        G8 gu[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = j0 + u * 64 + lane;
            gu[u] = g < g_end ? load_g8<DT, VEC>(row, g * 8, V) : G8{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = j0 + u * 64 + lane;
            const bool gin = g < g_end;
            const bool full = gin && g * 8 + 8 <= V;
            uint32_t ntc = 0;  // COLLECT: ties in this group
            if (VEC && DT == SV_BF16 && !ranked && full) {
                // two entries per operation
                const uint32_t kc2 = kcut | (kcut << 16);
                const uint4 a = gu[u].a;
                uint32_t k2[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) k2[i] = keys2(word_of(a, i));
                store16(static_cast<uint16_t*>(orow) + g * 8,
                        make_uint4(keep2(a.x, k2[0], kc2), keep2(a.y, k2[1], kc2), keep2(a.z, k2[2], kc2),
                                   keep2(a.w, k2[3], kc2)));
                if (!COLLECT) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t x = k2[i] ^ ks2;
                    ntc += ((x & 0xffffu) == 0u ? 1u : 0u) + ((x >> 16) == 0u ? 1u : 0u);
                }
            }
            if (COLLECT) {
                // number this group's ties after those of the lanes before it
                if (gin && !(VEC && DT == SV_BF16 && full)) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        ntc += (g * 8 + e < V && key_of<DT>(bits_of<DT>(gu[u], e)) == sel.kstar) ? 1u : 0u;
                }
                if (__ballot(ntc != 0u) != 0ull) {
                    const uint32_t incl = wave_incl_scan_t<uint32_t>(ntc);
                    uint32_t r = running + incl - ntc;
                    running += (uint32_t)__shfl((int)incl, 63, 64);
                    if (ntc != 0u) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if (g * 8 + e < V && key_of<DT>(bits_of<DT>(gu[u], e)) == sel.kstar) {
                                if (r < cap) list[r] = (uint32_t)(g * 8 + e);
                                ++r;
                            }
                        }
                    }
                }
                if (VEC && DT == SV_BF16 && full) continue;
            }
            uint32_t bits[8];
            bool keep[8], tie[8];
            uint32_t nt = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bits[e] = bits_of<DT>(gu[u], e);
                const uint32_t key = key_of<DT>(bits[e]);
                keep[e] = ranked ? key > sel.kstar : key >= kcut;
                tie[e] = ranked && gin && g * 8 + e < V && key == sel.kstar;
                nt += tie[e] ? 1u : 0u;
            }
            if (ranked && __ballot(nt != 0u) != 0ull) {  // ties in this group of the wave: rank them in index order
                const uint32_t incl = wave_incl_scan_t<uint32_t>(nt);
                uint32_t rank = running + incl - nt;
                running += (uint32_t)__shfl((int)incl, 63, 64);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (tie[e]) keep[e] = rank++ < sel.need;
            }
            if (!gin) continue;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (!keep[e]) bits[e] = kNegInf;
            if (VEC && full) {
                if constexpr (DT == SV_BF16) {
                    const uint4 w = make_uint4(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16),
                                               bits[4] | (bits[5] << 16), bits[6] | (bits[7] << 16));
                    store16(static_cast<uint16_t*>(orow) + g * 8, w);
                } else {
                    store16(static_cast<uint32_t*>(orow) + g * 8, make_uint4(bits[0], bits[1], bits[2], bits[3]));
                    store16(static_cast<uint32_t*>(orow) + g * 8 + 4, make_uint4(bits[4], bits[5], bits[6], bits[7]));
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (g * 8 + e >= V) continue;
                    if constexpr (DT == SV_BF16) static_cast<uint16_t*>(orow)[g * 8 + e] = (uint16_t)bits[e];
                    else static_cast<uint32_t*>(orow)[g * 8 + e] = bits[e];
                }
            }
        }
    }
    return running;
}

// The ties before this wave's run, from sm.tw (after a barrier).
__device__ __forceinline__ uint32_t ties_before(const StdSmall& sm)
{
    const int wv = (int)threadIdx.x >> 6;
    uint32_t s = 0;
    for (int w = 0; w < wv; ++w) s += sm.tw[w];
    return s;
}

// ------------------------------------------------------------ kernels

template <int DT, bool VEC, bool NUCLEUS>
__global__ __launch_bounds__(StdShape<NUCLEUS>::kSThreads) void k_standardize(const StdParams sp)
{
    const int V = sp.V;
    const size_t es = DT == SV_BF16 ? 2 : 4;
    const void* row = static_cast<const char*>(sp.in) + (size_t)blockIdx.x * V * es;
    void* orow = static_cast<char*>(sp.out) + (size_t)blockIdx.x * V * es;
    const Run run((V + 7) / 8, StdShape<NUCLEUS>::kSWaves);

    __shared__ uint32_t h_cnt[kBins];
    __shared__ double h_mass[NUCLEUS ? kBins : 1];
    __shared__ uint32_t h_tot[256];
    __shared__ StdSmall sm;

    Sel sel{NUCLEUS ? sp.top_p >= 1.0 : sp.k >= V, 0u, 0u};
    if (!sel.keep_all) sel = radix_select<DT, VEC, NUCLEUS>(sp, row, run, h_cnt, h_mass, h_tot, sm);
    const uint32_t tb = sel.keep_all ? 0u : ties_before(sm);
    const uint32_t tw = sel.keep_all ? 0u : sm.tw[threadIdx.x >> 6];
    write_row<DT, VEC>(sp, row, orow, run, sel, tb, tw);
}

// bf16 rows: the full 16-bit histogram (see the file comment).
template <bool VEC, bool NUCLEUS>
__global__ __launch_bounds__(kHThreads) void k_standardize_b16(const StdParams sp)
{
    constexpr int U = unroll_of<SV_BF16, VEC>();
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int V = sp.V;
    const void* row = static_cast<const uint16_t*>(sp.in) + (size_t)blockIdx.x * V;
    void* orow = static_cast<uint16_t*>(sp.out) + (size_t)blockIdx.x * V;
    const Run run((V + 7) / 8, kHWaves);

    __shared__ __align__(16) uint32_t hist[kHWords];  // key k: bits 16 (k & 1) .. +15 of word k >> 1
    __shared__ double rmass[NUCLEUS ? kHWords / 32 : 1];  // nucleus: mass of each range of 32 words
    __shared__ StdSmall sm;

    Sel sel{NUCLEUS ? sp.top_p >= 1.0 : sp.k >= V, 0u, 0u};
    uint32_t tb = 0, tw = 0;
    if (!sel.keep_all) {
        for (int i = tid; i < kHWords / 4; i += kHThreads) reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        auto count_key = [&](uint32_t key) { atomicAdd(&hist[key >> 1], (key & 1u) ? 0x10000u : 1u); };
        uint32_t kmax2 = 0, kmax1 = 0;  // nucleus: the largest key seen (packed pairs, single entries)
        for (int j0 = run.g_begin; j0 < run.g_end; j0 += U * 64) {  // uniform trip count
            G8 gu[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = j0 + u * 64 + lane;
                gu[u] = g < run.g_end ? load_g8<SV_BF16, VEC>(row, g * 8, V) : G8{};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = j0 + u * 64 + lane;
                if (g >= run.g_end) continue;
                if (g * 8 + 8 <= V) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t k2 = keys2(word_of(gu[u].a, i));
                        count_key(k2 & 0xffffu);
                        count_key(k2 >> 16);
                        if (NUCLEUS)
                            kmax2 = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, kmax2),
                                                                                          __builtin_bit_cast(u16x2, k2)));
                    }
                } else {
                    for (int e = 0; g * 8 + e < V; ++e) {
                        const uint32_t key = key_of<SV_BF16>(bits_of<SV_BF16>(gu[u], e));
                        count_key(key);
                        kmax1 = max(kmax1, key);
                    }
                }
            }
        }
        if (NUCLEUS) {
            uint32_t km = max(max(kmax2 & 0xffffu, kmax2 >> 16), kmax1);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) km = max(km, (uint32_t)__shfl_xor((int)km, o, 64));
            if (lane == 0) sm.kmax[tid >> 6] = km;  // published by the barrier below
        }
        __syncthreads();

        // thread t takes keys 65535 - 64 t down to 65472 - 64 t (words
        // 32767 - 32 t down to 32736 - 32 t): their count and mass, then a
        // workgroup scan in thread order; the crossing thread walks its keys
        // from the top
        const int w_lo = kHWords - 32 * (tid + 1);
        uint4 cw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) cw[i] = reinterpret_cast<const uint4*>(hist + w_lo)[i];
        auto cnt_at = [&](int j) -> uint32_t {  // j = 0 .. 63: key 65535 - 64 t - j
            const int wi = 31 - (j >> 1);
            const uint32_t w = word_of(cw[wi >> 2], wi & 3);
            return (j & 1) ? (w & 0xffffu) : (w >> 16);
        };
        uint32_t c_loc = 0;
#pragma unroll
        for (int j = 65536 / kHThreads - 1; j >= 0; --j) c_loc += cnt_at(j);  // 64 keys per thread
        // the row maximum: the largest key the counting pass saw
        double m = 0.0;
        if (NUCLEUS) {
            uint32_t km = 0;
            for (int w = 0; w < kHWaves; ++w) km = max(km, sm.kmax[w]);
            m = (double)value_of_key<SV_BF16>(km);
        }
        auto mass_of = [&](uint32_t key, uint32_t n) -> double {
            const float z = value_of_key<SV_BF16>(key);
            return z > -INFINITY ? (double)n * exp2_fast(((double)z - m) * sp.cd) : 0.0;
        };
        auto cnt_lds = [&](uint32_t key) -> uint32_t { return (hist[key >> 1] >> (16u * (key & 1u))) & 0xffffu; };
        double m_loc = 0.0;
        if (NUCLEUS) {
            // the mass of every thread's 32 words, computed across the whole
            // workgroup word by word (consecutive threads on consecutive
            // words, so the exponentials of the populated keys are spread
            // over all waves), each range of 32 words summed by half a wave
            for (int i = 0; i < kHWords / kHThreads; ++i) {
                const uint32_t wk = (uint32_t)(i * kHThreads + tid);
                const uint32_t w = hist[wk];
                double ms = 0.0;
                if (__ballot(w != 0u) != 0ull) {  // most words of the key space are empty
                    if (w >> 16) ms += mass_of(2u * wk + 1u, w >> 16);
                    if (w & 0xffffu) ms += mass_of(2u * wk, w & 0xffffu);
                    ms = half_wave_sum(ms);
                }
                if ((lane & 31) == 0) rmass[wk >> 5] = ms;
            }
            __syncthreads();
            m_loc = rmass[w_lo >> 5];
        }
        uint32_t c_tot, c_before;
        double m_tot = 0.0, m_before = 0.0;
        if (NUCLEUS) block_excl_scan2(c_loc, m_loc, sm.u, sm.d, &c_before, &m_before, &c_tot, &m_tot);
        else c_before = block_excl_scan<uint32_t>(c_loc, sm.u, &c_tot);
        if (c_tot != (uint32_t)V) {
            // some value occurs 65 536 times or more: a 16-bit counter wrapped
            __syncthreads();
            uint32_t* h_cnt = hist;
            double* h_mass = reinterpret_cast<double*>(hist + kBins);
            uint32_t* h_tot = hist + kBins + 2 * kBins;
            sel = radix_select<SV_BF16, VEC, NUCLEUS>(sp, row, run, h_cnt, h_mass, h_tot, sm);
            if (!sel.keep_all) {
                tb = ties_before(sm);
                tw = sm.tw[tid >> 6];
            }
        } else {
            const uint32_t rem_cnt = (uint32_t)min(sp.k, V);
            const double rem_mass = sp.top_p * m_tot;
            if (tid == 0) {
                sm.found = 0u;
                sm.tcross = 0xffffffffu;
            }
            __syncthreads();
            const bool cross = NUCLEUS ? (m_loc > 0.0 && m_before < rem_mass && rem_mass <= m_before + m_loc)
                                       : (c_before < rem_cnt && rem_cnt <= c_before + c_loc);
            // one thread's keys hold the crossing (the first, should rounding
            // let two claim it)
            if (cross) atomicMin(&sm.tcross, (uint32_t)tid);
            __syncthreads();
            if ((uint32_t)tid == sm.tcross) {
                sm.cb = c_before;
                sm.mb = m_before;
            }
            __syncthreads();
            const uint32_t tc = sm.tcross;
            if (tc != 0xffffffffu && tid < 64) {
                // wave 0 walks those 64 keys from the top, lane j on key
                // 65535 - 64 tc - j: the first key whose running count (mass)
                // reaches the target is the final key
                const uint32_t key = 65535u - 64u * tc - (uint32_t)lane;
                const uint32_t n = cnt_lds(key);
                uint64_t hit;
                uint32_t need = 0;
                if (NUCLEUS) {
                    const double mk = n ? mass_of(key, n) : 0.0;
                    const double incl = wave_incl_scan_t<double>(mk);
                    const double above = sm.mb + (incl - mk);
                    hit = __ballot(mk > 0.0 && rem_mass <= sm.mb + incl);
                    if (hit == 0ull) hit = 1ull << (63 - __builtin_clzll(__ballot(mk > 0.0)));  // rounding: the last key, whole
                    if (lane == __builtin_ctzll(hit)) {
                        const double q = ceil((rem_mass - above) / (mk / (double)n));
                        const bool crossed = rem_mass <= sm.mb + incl;
                        need = !crossed ? n : q < 1.0 ? 1u : q > (double)n ? n : (uint32_t)q;
                    }
                } else {
                    const uint32_t incl = wave_incl_scan_t<uint32_t>(n);
                    hit = __ballot(n > 0u && sm.cb + incl >= rem_cnt);
                    if (lane == __builtin_ctzll(hit)) need = rem_cnt - (sm.cb + incl - n);
                }
                if (lane == __builtin_ctzll(hit)) {
                    sm.kstar = key;
                    sm.need = need;
                    sm.partial = need < n ? 1u : 0u;
                    sm.found = 1u;
                }
            }
            __syncthreads();
            if (sm.found == 0u) {
                sel.keep_all = true;  // the running mass never reaches top_p (rounding): keep every entry
            } else {
                sel.kstar = sm.kstar;
                sel.need = sm.need;
                if (sm.partial) {
                    // write keeping every tie, each wave listing its ties
                    // (the histogram is no longer needed: its space holds
                    // the lists), then drop the ties past the kept ones
                    __syncthreads();
                    uint32_t* list = hist + (tid >> 6) * kTieCap;
                    const uint32_t n = write_row<SV_BF16, VEC, true>(sp, row, orow, run, sel, 0u, 0u, list, kTieCap);
                    if (lane == 0) sm.tw[tid >> 6] = n;
                    __syncthreads();
                    tb = ties_before(sm);
                    const uint32_t keep_here = sel.need > tb ? sel.need - tb : 0u;  // ties of this run kept
                    if (keep_here < n) {
                        if (n <= kTieCap) {
                            for (uint32_t r = keep_here + (uint32_t)lane; r < n; r += 64u)
                                static_cast<uint16_t*>(orow)[list[r]] = (uint16_t)0xff80u;
                        } else {
                            // more ties than the list holds: rewrite the run ranking them
                            // (entries at or above the final key are unchanged in orow, so
                            // this holds in place too)
                            write_row<SV_BF16, VEC>(sp, row, orow, run, sel, tb, n);
                        }
                    }
                    return;
                }
                // otherwise every tie is kept: tb = tw = 0 <= need
            }
        }
    }
    write_row<SV_BF16, VEC>(sp, row, orow, run, sel, tb, tw);
}

inline bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" int sv_standardize(int rows, int vocab, const void* logits, int dtype, int method, int k, float top_p,
                              float temperature, void* logits_out, void* stream)
{
    if (!logits || !logits_out) return SV_ERR_NULL_POINTER;
    if (rows < 1) return SV_ERR_BATCH;
    if (vocab < 1) return SV_ERR_VOCAB;
    if (dtype != SV_FP32 && dtype != SV_BF16) return SV_ERR_DTYPE;
    if (method != SV_TOPK && method != SV_TOPP) return SV_ERR_STANDARDIZE;
    if (method == SV_TOPK && k < 1) return SV_ERR_STANDARDIZE;
    if (method == SV_TOPP && !(top_p > 0.0f && top_p <= 1.0f)) return SV_ERR_STANDARDIZE;
    if (method == SV_TOPP && (!(temperature > 0.0f) || !std::isfinite(temperature))) return SV_ERR_TEMPERATURE;
    const size_t es = dtype == SV_BF16 ? 2 : 4;
    if (!aligned_to(logits, es) || !aligned_to(logits_out, es)) return SV_ERR_ALIGNMENT;
    StdParams sp;
    sp.in = logits;
    sp.out = logits_out;
    sp.V = vocab;
    sp.method = method;
    sp.k = k;
    sp.top_p = (double)top_p;
    sp.cd = method == SV_TOPP ? 1.4426950408889634 / (double)temperature : 0.0;
    const bool vec = aligned_to(logits, 16) && aligned_to(logits_out, 16) && ((size_t)vocab * es) % 16 == 0;
    hipStream_t s = (hipStream_t)stream;
    const bool nuc = method == SV_TOPP;
    const dim3 g(rows);
    if (dtype == SV_BF16) {
        const dim3 t(kHThreads);
        if (vec) {
            if (nuc) hipLaunchKernelGGL((k_standardize_b16<true, true>), g, t, 0, s, sp);
            else hipLaunchKernelGGL((k_standardize_b16<true, false>), g, t, 0, s, sp);
        } else {
            if (nuc) hipLaunchKernelGGL((k_standardize_b16<false, true>), g, t, 0, s, sp);
            else hipLaunchKernelGGL((k_standardize_b16<false, false>), g, t, 0, s, sp);
        }
    } else {
        const dim3 t(nuc ? StdShape<true>::kSThreads : StdShape<false>::kSThreads);
        if (vec) {
            if (nuc) hipLaunchKernelGGL((k_standardize<SV_FP32, true, true>), g, t, 0, s, sp);
            else hipLaunchKernelGGL((k_standardize<SV_FP32, true, false>), g, t, 0, s, sp);
        } else {
            if (nuc) hipLaunchKernelGGL((k_standardize<SV_FP32, false, true>), g, t, 0, s, sp);
            else hipLaunchKernelGGL((k_standardize<SV_FP32, false, false>), g, t, 0, s, sp);
        }
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
