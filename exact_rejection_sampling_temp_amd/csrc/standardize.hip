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
// One workgroup per row (512 threads for top-k, two rows per CU; 1024 for
// the nucleus).  The kept set is found by an MSB-first
// radix select over order-preserving integer keys of the logits (12-bit then
// 4-bit digits for bf16; 12, 12, 8 for fp32): a pass over the row builds the
// digit's histogram in LDS (element counts, and for nucleus the fp64 masses
// exp((z - max)/T)), a workgroup scan over the bins from the top finds the
// bin where the count (mass) crosses k (top_p times the row's mass), and
// the next pass refines inside that bin.  Entries equal to the final key
// are ties; the first ones in index order are kept (counted with a
// workgroup scan per round of the last pass).  Ties in value are ordered by
// index, so top-k keeps exactly min(k, V) entries.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "spec_verify.h"

namespace {

// workgroup size: 512 threads for top-k (two rows per CU), 1024 for the
// nucleus, whose fp64 mass atomics and polynomial need the registers
template <bool NUCLEUS>
struct StdShape {
    static constexpr int kSThreads = NUCLEUS ? 1024 : 512;
    static constexpr int kSWaves = kSThreads / 64;
    static constexpr int kBinsPerThread = 4096 / kSThreads;
};
constexpr int kMaxWaves = 16;
constexpr int kBins = 4096;  // 12-bit digits
constexpr int kUnroll = 4;  // groups of 8 entries per thread per histogram iteration

struct StdParams {
    const void* in;
    void* out;
    int V, method, k;
    double top_p;
    double cd;  // log2(e)/T
};

// Order-preserving keys: larger value <=> larger key; -0 is folded onto +0
// (equal values compare equal, their order is by index).
template <int DT>
__device__ __forceinline__ uint32_t key_of(uint32_t bits)
{
    if constexpr (DT == SV_BF16) {
        if (bits == 0x8000u) bits = 0u;
        return bits ^ ((bits & 0x8000u) ? 0xffffu : 0x8000u);
    } else {
        if (bits == 0x80000000u) bits = 0u;
        return bits ^ ((bits & 0x80000000u) ? 0xffffffffu : 0x80000000u);
    }
}
template <int DT>
__device__ __forceinline__ float value_of_key(uint32_t key)
{
    if constexpr (DT == SV_BF16) {
        const uint32_t bits = (key & 0x8000u) ? (key ^ 0x8000u) : (key ^ 0xffffu);
        return __uint_as_float(bits << 16);
    } else {
        const uint32_t bits = (key & 0x80000000u) ? (key ^ 0x80000000u) : (key ^ 0xffffffffu);
        return __uint_as_float(bits);
    }
}
template <int DT>
__device__ __forceinline__ float value_of_bits(uint32_t bits)
{
    if constexpr (DT == SV_BF16) return __uint_as_float(bits << 16);
    else return __uint_as_float(bits);
}

// 8 consecutive raw elements (bit patterns) starting at index base; entries
// at or past V are reported invalid.  VEC: 16-byte aligned rows.
template <int DT, bool VEC>
__device__ __forceinline__ void load8(const void* row, int base, int V, uint32_t (&bits)[8], bool (&ok)[8])
{
#pragma unroll
    for (int e = 0; e < 8; ++e) ok[e] = base + e < V;
    if constexpr (VEC) {
        if (base + 8 <= V) {
            if constexpr (DT == SV_BF16) {
                const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + base);
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) bits[e] = (ws[e >> 1] >> (16 * (e & 1))) & 0xffffu;
            } else {
                const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const float*>(row) + base);
                const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const float*>(row) + base + 4);
                bits[0] = a.x; bits[1] = a.y; bits[2] = a.z; bits[3] = a.w;
                bits[4] = b.x; bits[5] = b.y; bits[6] = b.z; bits[7] = b.w;
            }
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int i = min(base + e, V - 1);
        if constexpr (DT == SV_BF16) bits[e] = static_cast<const uint16_t*>(row)[i];
        else bits[e] = static_cast<const uint32_t*>(row)[i];
    }
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

// Exclusive scan over the workgroup in thread order; *total gets the sum.
template <typename T>
__device__ T block_excl_scan(T v, T* sm, T* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int kSWaves = (int)(blockDim.x >> 6);
    const T incl = wave_incl_scan_t(v);
    if (lane == 63) sm[w] = incl;
    __syncthreads();
    T before = T(0), all = T(0);
#pragma unroll
    for (int i = 0; i < kMaxWaves; ++i) {
        if (i >= kSWaves) break;
        const T s = sm[i];
        if (i < w) before += s;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

__device__ uint32_t block_max_u32(uint32_t v, uint32_t* sm)
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

template <int DT, bool VEC, bool NUCLEUS>
__global__ __launch_bounds__(StdShape<NUCLEUS>::kSThreads) void k_standardize(const StdParams sp)
{
    constexpr int kSThreads = StdShape<NUCLEUS>::kSThreads;
    constexpr int kBinsPerThread = StdShape<NUCLEUS>::kBinsPerThread;
    constexpr int KB = DT == SV_BF16 ? 16 : 32;
    constexpr int NPASS = DT == SV_BF16 ? 2 : 3;
    constexpr int kShift[3] = {KB - 12, DT == SV_BF16 ? 0 : 8, 0};
    constexpr int kDigit[3] = {12, DT == SV_BF16 ? 4 : 12, 8};
    constexpr bool nucleus = NUCLEUS;
    const int tid = (int)threadIdx.x;
    const int V = sp.V;
    const size_t es = DT == SV_BF16 ? 2 : 4;
    const void* row = static_cast<const char*>(sp.in) + (size_t)blockIdx.x * V * es;
    void* orow = static_cast<char*>(sp.out) + (size_t)blockIdx.x * V * es;
    const int ngroups = (V + 7) / 8;

    __shared__ uint32_t h_cnt[kBins];
    __shared__ double h_mass[kBins];
    __shared__ uint32_t sm_u[kMaxWaves];
    __shared__ double sm_d[kMaxWaves];
    __shared__ uint32_t sm_bin;
    __shared__ uint32_t sm_above_cnt;
    __shared__ double sm_above_mass;

    // the row maximum (nucleus masses are taken relative to it)
    double m = 0.0;
    if (nucleus) {
        uint32_t mk = 0;
        for (int g = tid; g < ngroups; g += kSThreads) {
            uint32_t bits[8];
            bool ok[8];
            load8<DT, VEC>(row, g * 8, V, bits, ok);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (ok[e]) mk = max(mk, key_of<DT>(bits[e]));
        }
        m = (double)value_of_key<DT>(block_max_u32(mk, sm_u));
    }

    // top-k with k >= V, and the nucleus of the whole mass, keep every entry
    bool keep_all = nucleus ? sp.top_p >= 1.0 : sp.k >= V;
    uint32_t prefix = 0;
    uint32_t rem_cnt = (uint32_t)min(sp.k, V);
    double rem_mass = 0.0;
    for (int ps = 0; ps < NPASS && !keep_all; ++ps) {
        const int shift = kShift[ps], dbits = kDigit[ps];
        const uint32_t dmask = (1u << dbits) - 1u;
        for (int i = tid; i < kBins; i += kSThreads) {
            h_cnt[i] = 0u;
            h_mass[i] = 0.0;
        }
        __syncthreads();
        for (int g0 = tid; g0 < ngroups; g0 += kUnroll * kSThreads) {
            uint32_t bitsu[kUnroll][8];
            bool oku[kUnroll][8];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {  // every load of the iteration in flight at once
                const int g = g0 + u * kSThreads;
                if (g < ngroups) {
                    load8<DT, VEC>(row, g * 8, V, bitsu[u], oku[u]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) { bitsu[u][e] = 0u; oku[u][e] = false; }
                }
            }
#pragma unroll
            for (int ue = 0; ue < kUnroll * 8; ++ue) {
                const int e = ue & 7;
                const uint32_t (&bits)[8] = bitsu[ue >> 3];
                const bool (&ok)[8] = oku[ue >> 3];
                const uint32_t key = key_of<DT>(bits[e]);
                const uint32_t hi = shift + dbits >= 32 ? 0u : (key >> (shift + dbits));
                if (!ok[e] || hi != prefix) continue;
                const uint32_t bin = (key >> shift) & dmask;
                atomicAdd(&h_cnt[bin], 1u);
                if (nucleus) {
                    const float z = value_of_bits<DT>(bits[e]);
                    if (z > -INFINITY) atomicAdd(&h_mass[bin], exp2_fast(((double)z - m) * sp.cd));
                }
            }
        }
        __syncthreads();
        // bins from the top: thread t takes bins 4095-4t .. 4092-4t
        uint32_t c_loc = 0;
        double m_loc = 0.0;
#pragma unroll
        for (int i = 0; i < kBinsPerThread; ++i) {
            const int b = kBins - 1 - (kBinsPerThread * tid + i);
            c_loc += h_cnt[b];
            m_loc += h_mass[b];
        }
        uint32_t c_tot;
        double m_tot;
        uint32_t c_before = block_excl_scan<uint32_t>(c_loc, sm_u, &c_tot);
        double m_before = block_excl_scan<double>(m_loc, sm_d, &m_tot);
        if (ps == 0 && nucleus) rem_mass = sp.top_p * m_tot;  // the row's mass, summed once
        if (tid == 0) sm_bin = 0xffffffffu;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kBinsPerThread; ++i) {
            const int b = kBins - 1 - (kBinsPerThread * tid + i);
            const uint32_t hc = h_cnt[b];
            const double hm = h_mass[b];
            const bool cross = nucleus ? (hc > 0 && m_before < rem_mass && rem_mass <= m_before + hm)
                                       : (c_before < rem_cnt && rem_cnt <= c_before + hc);
            if (cross) {
                sm_bin = (uint32_t)b;
                sm_above_cnt = c_before;
                sm_above_mass = m_before;
            }
            c_before += hc;
            m_before += hm;
        }
        __syncthreads();
        const uint32_t bin = sm_bin;
        if (bin == 0xffffffffu) {
            keep_all = true;  // the running mass never reaches top_p (rounding): keep every entry
        } else {
            prefix = (prefix << dbits) | bin;
            rem_cnt -= sm_above_cnt;
            rem_mass -= sm_above_mass;
        }
        __syncthreads();
    }

    // ties at the final key: how many of them, in index order, are kept
    const uint32_t kstar = prefix;
    uint32_t need = rem_cnt;
    if (!keep_all && nucleus) {
        const double wt = exp2_fast(((double)value_of_key<DT>(kstar) - m) * sp.cd);
        const double n = ceil(rem_mass / wt);
        need = n < 1.0 ? 1u : (n > 4294967295.0 ? 0xffffffffu : (uint32_t)n);
    }

    // write the row: kept entries as they are, the rest -inf
    const int nrounds = (ngroups + kSThreads - 1) / kSThreads;
    uint32_t running = 0;
    for (int r = 0; r < nrounds; ++r) {
        const int g = r * kSThreads + tid;
        uint32_t bits[8];
        bool ok[8];
        if (g < ngroups) {
            load8<DT, VEC>(row, g * 8, V, bits, ok);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) { bits[e] = 0u; ok[e] = false; }
        }
        uint32_t nt = 0;
        uint32_t keyv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            keyv[e] = key_of<DT>(bits[e]);
            if (ok[e] && keyv[e] == kstar) ++nt;
        }
        uint32_t tot;
        uint32_t rank = running + block_excl_scan<uint32_t>(nt, sm_u, &tot);
        running += tot;
        if (g < ngroups) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (!ok[e]) continue;
                bool keep = keep_all || keyv[e] > kstar;
                if (!keep && keyv[e] == kstar) keep = rank++ < need;
                const int i = g * 8 + e;
                if constexpr (DT == SV_BF16)
                    static_cast<uint16_t*>(orow)[i] = keep ? (uint16_t)bits[e] : (uint16_t)0xff80u;
                else
                    static_cast<uint32_t*>(orow)[i] = keep ? bits[e] : 0xff800000u;
            }
        }
    }
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
    const bool vec = aligned_to(logits, 16) && ((size_t)vocab * es) % 16 == 0;
    hipStream_t s = (hipStream_t)stream;
    const bool nuc = method == SV_TOPP;
    const dim3 g(rows), t(nuc ? StdShape<true>::kSThreads : StdShape<false>::kSThreads);
    if (dtype == SV_BF16) {
        if (vec) {
            if (nuc) hipLaunchKernelGGL((k_standardize<SV_BF16, true, true>), g, t, 0, s, sp);
            else hipLaunchKernelGGL((k_standardize<SV_BF16, true, false>), g, t, 0, s, sp);
        } else {
            if (nuc) hipLaunchKernelGGL((k_standardize<SV_BF16, false, true>), g, t, 0, s, sp);
            else hipLaunchKernelGGL((k_standardize<SV_BF16, false, false>), g, t, 0, s, sp);
        }
    } else {
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
