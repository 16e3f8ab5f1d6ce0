/* Bounds check of the launch geometry and the workspace layout, on the CPU
 * (test side only).
 *
 * Built by tests/test_layout_check.py with hipcc into a host program that
 * includes the library's source, so that it calls the library's own
 * make_layout and make_plan and the block decodes its kernels use
 * (row_block, helper_task, wave_sub, beta_block, rest_task).  Over a sweep
 * of shapes (batch, gamma, vocab, dtypes, modes) including the extremes, it
 * checks that every workgroup a launch would start maps to work inside the
 * problem, that every workspace array the kernels index with those
 * coordinates fits inside its region, that the regions are 256-byte aligned
 * and disjoint, and that the total is sv_workspace_bytes.  No kernel runs
 * and no GPU is needed.  Prints the number of failed checks.
 */
#include "../exact_rejection_sampling_temp_amd/csrc/spec_verify.hip"

#include <cstdio>
#include <vector>

static long long g_checks = 0, g_failed = 0;

#define CHECK(cond, ...)                                                   \
    do {                                                                   \
        ++g_checks;                                                        \
        if (!(cond)) {                                                     \
            if (++g_failed <= 20) {                                        \
                std::fprintf(stderr, "FAILED %s: ", #cond);                \
                std::fprintf(stderr, __VA_ARGS__);                         \
                std::fprintf(stderr, "\n");                                \
            }                                                              \
        }                                                                  \
    } while (0)

// block indices worth checking in a grid of n: both ends and around every
// multiple of `step` near them, plus a spread of interior ones
static std::vector<long long> probe(long long n, long long step)
{
    std::vector<long long> v;
    for (long long i : {0LL, 1LL, 2LL, n / 2, n - 2, n - 1})
        if (i >= 0 && i < n) v.push_back(i);
    for (long long m = step; m < n && m < 64 * step; m += step)
        for (long long d : {-1LL, 0LL, 1LL})
            if (m + d >= 0 && m + d < n) v.push_back(m + d);
    for (long long i = 0; i < 64; ++i) v.push_back((n - 1) * i / 63);
    return v;
}

static void check_shape(int B, int gamma, int V, int ldt, int pdt, bool greedy, bool tele)
{
    const int G1 = gamma + 1;
    const size_t lsz = ldt == SV_BF16 ? 2 : 4, psz = pdt == SV_BF16 ? 2 : 4;
    const Layout L = make_layout(B, gamma, V);
    const Plan q = make_plan(B, gamma, V, ldt, greedy, tele);
    const size_t total = sv_workspace_bytes(B, gamma, V);
    CHECK(total == L.total, "B=%d g=%d V=%d: sv_workspace_bytes %zu, layout %zu", B, gamma, V, total, L.total);

    // regions: 256-byte aligned, in order, disjoint, each as large as its
    // kernels index it
    const size_t rows = (size_t)B * G1;
    struct Region { const char* name; size_t off, need; };
    const Region reg[] = {
        {"ctl", L.ctl_off, sizeof(SeqCtl) * (size_t)B},
        {"cnt1", L.cnt1_off, sizeof(uint64_t) * rows},
        {"ready", L.ready_off, sizeof(uint32_t) * (size_t)B},
        {"ready_cnt", L.rcnt_off, sizeof(uint32_t)},
        {"part1", L.part1_off, 2 * sizeof(uint64_t) * rows * (size_t)q.nch1},
        {"stats", L.stats_off, sizeof(RowStat) * rows},
        {"sub", L.sub_off, sizeof(SubSum) * (size_t)B * (size_t)L.nsub},
        {"bpart", L.bpart_off, sizeof(double) * (size_t)B * (size_t)gamma * (size_t)L.nchb},
    };
    const int nreg = (int)(sizeof(reg) / sizeof(reg[0]));
    for (int i = 0; i < nreg; ++i) {
        const size_t end = i + 1 < nreg ? reg[i + 1].off : L.total;
        CHECK(reg[i].off % 256 == 0, "B=%d g=%d V=%d: %s at %zu", B, gamma, V, reg[i].name, reg[i].off);
        CHECK(reg[i].off + reg[i].need <= end, "B=%d g=%d V=%d: %s needs %zu bytes at %zu, next region at %zu",
              B, gamma, V, reg[i].name, reg[i].need, reg[i].off, end);
    }
    CHECK(L.control_bytes == L.part1_off, "control words end where the partials start");
    CHECK(q.nch1 <= L.nch1_max, "B=%d g=%d V=%d: nch1 %d > nch1_max %d", B, gamma, V, q.nch1, L.nch1_max);
    CHECK(L.nch2 * kChunk2 >= V && (L.nch2 - 1) * kChunk2 < V, "draw chunks cover the row exactly");
    CHECK(L.nsub == L.nch2 * kWaves, "sub-chunks per sequence");
    CHECK(L.nchb * kChunkB >= V && (L.nchb - 1) * kChunkB < V, "telemetry chunks cover the row exactly");

    if (q.status != SV_OK) {
        // refused: one of the limits really is passed
        const bool over = q.nch1 > 0xffff || q.gridh > INT_MAX || q.grid2 > INT_MAX || q.gridb > INT_MAX ||
                          (!greedy && B > kMaxListed);
        CHECK(over, "B=%d g=%d V=%d: refused without a limit passed", B, gamma, V);
        return;
    }
    CHECK(q.gridh <= INT_MAX && q.grid2 <= INT_MAX && q.gridb <= INT_MAX, "grids fit an int");

    if (q.small) {
        // k_small: one wave per sequence; k_tiny: four (rows of 16 lanes) or
        // eight (rows of 8) per wave, every entry of a row in a lane of its own
        const long long per = q.tiny ? (64LL / q.tiny_lanes) * kWaves : (long long)kWaves;
        CHECK(q.seqs_per_wg == per, "sequences per workgroup");
        CHECK(q.grid_small * per >= B && (q.grid_small - 1) * per < B, "B=%d: small grid %lld", B, q.grid_small);
        CHECK(V <= (q.tiny ? q.tiny_lanes : kSmallV), "V=%d on the one-launch path", V);
        CHECK(!q.tiny || q.tiny_lanes == 16 || gamma + 1 <= 8, "an 8-lane row holds the gamma + 1 uniforms");
        CHECK(!q.tiny || gamma + 1 <= 16, "the tiny path holds at most 16 rows per sequence");
        return;
    }

    // the row stage (sample and greedy): every workgroup has a position,
    // sequence and chunk inside the problem, and its chunk starts inside the row
    const int CH = ldt == SV_BF16 && !q.half_chunks ? kChunkBf16 : kChunkFp32;
    CHECK(!q.half_chunks || (greedy && ldt == SV_BF16 &&
                             (long long)B * ((V + kChunkBf16 - 1) / kChunkBf16) <= kHalfChunkBlocks),
          "half-size chunks only for greedy bf16 calls of small batches");
    CHECK((long long)q.nch1 * CH >= V && (long long)(q.nch1 - 1) * CH < V, "row chunks cover the row exactly");
    CHECK(q.nch1 <= L.nch1_max, "row chunks within the partial region's sizing");
    for (long long bid : probe(q.grid1, q.nch1)) {
        const RowBlock rb = row_block((uint32_t)bid, q.nch1, B);
        CHECK(rb.k >= 0 && rb.k <= gamma && rb.b >= 0 && rb.b < B && rb.c >= 0 && rb.c < q.nch1,
              "B=%d g=%d V=%d: row block %lld -> k=%d b=%d c=%d", B, gamma, V, bid, rb.k, rb.b, rb.c);
        CHECK((long long)rb.c * CH < V, "chunk %d starts past the row (V=%d)", rb.c, V);
        const size_t row = (size_t)rb.b * G1 + rb.k;
        CHECK(2 * sizeof(uint64_t) * (row * q.nch1 + rb.c + 1) <= reg[4].need, "partial slot in its region");
        CHECK((row + 1) * lsz * (size_t)V <= rows * lsz * (size_t)V, "target row inside the logits");
    }
    // and the decode is one to one on consecutive indices
    for (long long bid : probe(q.grid1 - 1, q.nch1)) {
        const RowBlock a = row_block((uint32_t)bid, q.nch1, B), b2 = row_block((uint32_t)(bid + 1), q.nch1, B);
        const long long ia = ((long long)a.k * B + a.b) * q.nch1 + a.c, ib = ((long long)b2.k * B + b2.b) * q.nch1 + b2.c;
        CHECK(ia == bid && ib == bid + 1, "row decode is the inverse of (k * B + b) * nch1 + c at %lld", bid);
    }
    if (greedy) {
        CHECK(q.grid2 == B, "greedy: one draw workgroup per sequence");
        return;
    }
    if (q.helpers && q.fine) {
        // one helper per sub-chunk, wave w on group w of it
        CHECK((long long)B * L.nsub <= kFineHelpers, "fine helpers only for small batches");
        CHECK(q.gridh == q.grid1 + (long long)B * L.nsub, "fine helpers follow the row blocks");
        CHECK(q.grid2 == B, "last launch: one workgroup per sequence");
        std::vector<int> seen((size_t)B * L.nsub, 0);
        for (long long j = 0; j < (long long)B * L.nsub; ++j) {
            const DrawTask t = fine_task((int)j, L.nsub);
            CHECK(t.r >= 0 && t.r < B && t.c2 >= 0 && t.c2 < L.nsub, "fine helper %lld -> r=%d s=%d", j, t.r, t.c2);
            if (t.r >= 0 && t.r < B && t.c2 >= 0 && t.c2 < L.nsub) ++seen[(size_t)t.r * L.nsub + t.c2];
            for (int w = 0; w < kWaves; ++w) {
                const long long grp = (long long)t.c2 * kSubPerWave + w;  // its first entry may lie past V (then no load)
                CHECK(grp >= 0 && grp < (long long)L.nsub * kSubPerWave, "fine helper %lld wave %d -> group %lld", j, w, grp);
            }
            CHECK(sizeof(SubSum) * ((size_t)(B - 1) * L.nsub + t.c2 + 1) <= reg[6].need, "draw sums in their region");
        }
        for (size_t k = 0; k < seen.size(); ++k) CHECK(seen[k] == 1, "sub-chunk task %zu taken %d times", k, seen[k]);
    } else if (q.helpers) {
        CHECK((long long)B * L.nsub > kFineHelpers, "chunk helpers only for large batches");
        CHECK(q.gridh == q.grid1 + (long long)B * L.nch2, "helpers follow the row blocks");
        CHECK(q.grid2 == B, "last launch: one workgroup per sequence");
        for (long long j : probe((long long)B * L.nch2, L.nch2)) {
            const DrawTask t = helper_task((int)j, L.nch2);
            CHECK(t.r >= 0 && t.r < B && t.c2 >= 0 && t.c2 < L.nch2, "helper %lld -> r=%d c2=%d", j, t.r, t.c2);
            for (int w = 0; w < kWaves; ++w) {
                const int sidx = wave_sub(t.c2, w);
                CHECK(sidx >= 0 && sidx < L.nsub, "helper %lld wave %d -> sub-chunk %d of %d", j, w, sidx, L.nsub);
                CHECK(sizeof(SubSum) * ((size_t)(B - 1) * L.nsub + sidx + 1) <= reg[6].need, "draw sums in their region");
            }
        }
    } else {
        // telemetry: the sweep, then k_rest_sample
        CHECK(q.gridb == (long long)B * gamma * L.nchb, "telemetry sweep grid");
        for (long long bid : probe(q.gridb, L.nchb)) {
            const BetaBlock bb = beta_block((uint32_t)bid, L.nchb, gamma);
            CHECK(bb.b >= 0 && bb.b < B && bb.i >= 0 && bb.i < gamma && bb.c >= 0 && bb.c < L.nchb,
                  "beta block %lld -> b=%d i=%d c=%d", bid, bb.b, bb.i, bb.c);
            CHECK((long long)bb.c * kChunkB < V, "telemetry chunk starts inside the row");
            CHECK(sizeof(double) * (((size_t)bb.b * gamma + bb.i) * L.nchb + bb.c + 1) <= reg[7].need,
                  "telemetry slot in its region");
            CHECK(((size_t)bb.b * gamma + bb.i + 1) * psz * (size_t)V <= (size_t)B * gamma * psz * (size_t)V,
                  "draft row inside the draft probabilities");
        }
        CHECK(q.grid2 == (long long)B * L.nch2, "k_rest_sample grid");
        const bool all = (long long)B * L.nch2 <= 1 << 16;
        std::vector<int> seen(all ? (size_t)B * L.nch2 : 0, 0);
        for (long long i : all ? std::vector<long long>() : probe(q.grid2, B)) {
            const RestTask rt = rest_task((int)i, B, L.nch2);
            CHECK(rt.r >= 0 && rt.r < B && rt.j >= 0 && rt.j < (L.nch2 > 1 ? L.nch2 : 1), "rest %lld -> r=%d j=%d", i, rt.r, rt.j);
        }
        if (all) {
            // every (rank, workgroup) pair exactly once
            for (long long i = 0; i < q.grid2; ++i) {
                const RestTask rt = rest_task((int)i, B, L.nch2);
                const bool in = rt.r >= 0 && rt.r < B && rt.j >= 0 && rt.j < L.nch2;
                CHECK(in, "rest %lld -> r=%d j=%d", i, rt.r, rt.j);
                if (in) ++seen[(size_t)rt.r * L.nch2 + rt.j];
            }
            for (size_t k = 0; k < seen.size(); ++k) CHECK(seen[k] == 1, "rest task %zu taken %d times", k, seen[k]);
        }
    }
}

// The first launch's occupancy cap: 3..8 row blocks per CU, growing with the
// blocks of one position; the dynamic LDS lets exactly that many workgroups
// share a CU (static LDS up to 200 bytes, allocation granules up to 1280).
static void check_occupancy_cap()
{
    for (int h : {kSampleHalfPositions, kGreedyHalfPositions})
        for (int n_cu : {1, 80, 256, 304}) {
            int prev = 0;
            for (long long bpp = 1; bpp < (1LL << 26); bpp = bpp * 3 / 2 + 1) {
                const int w = row_wgs_per_cu(bpp, n_cu, h);
                CHECK(w >= kMinRowWgsPerCu && w <= kMaxRowWgsPerCu && w >= prev, "h=%d n_cu=%d bpp=%lld -> %d", h,
                      n_cu, bpp, w);
                // between the bounds, w = ceil(h/2 * bpp / n_cu)
                if (w > kMinRowWgsPerCu && w < kMaxRowWgsPerCu)
                    CHECK(2LL * (w - 1) * n_cu < h * bpp && h * bpp <= 2LL * w * n_cu, "h=%d n_cu=%d bpp=%lld", h,
                          n_cu, bpp);
                prev = w;
            }
        }
    // 256 CUs: c4 (256 sequences x 10 chunks) uncapped; c3 and c5 (512 blocks
    // a position) at 3 in sample mode and 4 in greedy mode
    CHECK(row_wgs_per_cu(2560, 256, kSampleHalfPositions) == 8 && row_wgs_per_cu(2560, 256, kGreedyHalfPositions) == 8 &&
              row_wgs_per_cu(512, 256, kSampleHalfPositions) == 3 && row_wgs_per_cu(512, 256, kGreedyHalfPositions) == 4,
          "the measured shapes");
    for (int lds : {65536, 163840}) {
        CHECK(cap_lds_bytes(kMaxRowWgsPerCu, lds, lds) == 0u, "no cap at 8");
        for (int w = kMinRowWgsPerCu; w < kMaxRowWgsPerCu; ++w) {
            const long long d = cap_lds_bytes(w, lds, lds);
            const long long held = (d + 200 + 1279) / 1280 * 1280;
            CHECK(d > 0 && w * held <= lds && (w + 1) * d > lds, "lds=%d w=%d dyn=%lld", lds, w, d);
        }
        CHECK(cap_lds_bytes(3, lds, 1024) == 0u, "above the per-workgroup limit: no cap");
        for (int w = kMinRowWgsPerCu; w < kMaxRowWgsPerCu; ++w) {
            const long long d = cap_lds_bytes(w, lds, 65536);
            CHECK(d == 0 || d + 200 <= 65536, "dynamic and static LDS within a 64 KiB workgroup limit (w=%d)", w);
        }
    }
}

int main()
{
    check_occupancy_cap();
    const int batches[] = {1, 2, 3, 7, 64, 255, 256, 1231, 4096, 100000, kMaxListed, kMaxListed + 1};
    const int gammas[] = {1, 2, 4, 8, 15, 16, 62, 63};
    const int vocabs[] = {1, 7, 8, 16, 17, 512, 513, 8191, 8192, 8193, 16383, 16384, 16385, 32000, 128256,
                          152064, 256000, 1 << 20, 65535 * 16384, 65535 * 16384 + 1};
    for (int B : batches)
        for (int g : gammas)
            for (int V : vocabs)
                for (int ldt : {SV_FP32, SV_BF16})
                    for (int mode = 0; mode < 3; ++mode) {
                        // (shapes whose workspace would pass size_t stay out)
                        if ((double)B * (g + 1) * (double)V > 4e12) continue;
                        const int pdt = ldt == SV_BF16 && mode != 1 ? SV_BF16 : SV_FP32;
                        check_shape(B, g, V, ldt, pdt, mode == 1, mode == 2);
                    }
    std::printf("layout check: %lld checks, %lld failed checks\n", g_checks, g_failed);
    return g_failed ? 1 : 0;
}
