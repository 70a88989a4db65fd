// Where the time of one LDS-DMA kernel launch goes, workgroup by workgroup.
//
// Small shapes take a few microseconds per launch whatever their flop count,
// and this program breaks that time down.  It builds the library's kernel with
// its timeline hooks defined: every workgroup stamps the GPU's constant-rate
// real-time counter (s_memrealtime) at entry, when the first ring stage is in
// LDS, when its last unit's K loop ends, when that unit's C stores are issued,
// and at exit (after its stores have completed).  The stamps stay in registers
// until exit, where thread 0 writes them with ordinary vector stores: one
// record per workgroup per launch, at the launch count the workgroup read at
// entry, so launches run back to back with nothing between them.
//
// Per shape (the configuration the library's AUTO dispatch picks for it, on the
// same rotated input sets the bench uses), after 3 untimed launches, `--reps`
// back-to-back launches are timed with HIP events and recorded; each reported
// phase is the median over launches of:
//   ramp_us         the last workgroup's entry after the first one's;
//   first_stage_us  entry to the first stage in LDS (median over workgroups);
//   k_loop_us       first stage to the end of the last unit's K loop (median);
//   epilogue_us     ReLU, rounding and C stores issued (median);
//   store_drain_us  stores issued to stores complete at exit (median);
//   span_us         first entry to last exit;
//   gap_us          last exit of a launch to first entry of the next;
// and the distribution of workgroup exit times after the launch's first entry
// (over all workgroups and launches, and its median per XCD), with where the
// late workgroups ran: each workgroup also records its XCD, shader engine and
// CU (the XCC_ID and HW_ID hardware registers) and its last tile, and the
// program lists, per XCD, the shader engine whose workgroups exit last, and
// every workgroup whose median exit is more than 15% after the median
// workgroup's, with its tile origin and where its columns start in a B row.
// A sampled check of C against fp64 sums follows each shape.
//
// Usage: kernel_timeline [--reps N] [--shape NAME]
// Output: one JSON line per shape, then {"checked": true} (exit status 1 on a
// mismatch).
#define GEMM_RELU_TIMELINE 1

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

namespace timeline {
__device__ unsigned* g_count;             // per workgroup: launches recorded so far
__device__ unsigned long long* g_rec;     // [launch][workgroup][7]: real-time stamps, placement, tile
__device__ unsigned g_max_launches;
}  // namespace timeline

#define GEMM_RELU_TIMELINE_BEGIN                                                                    \
    unsigned long long gr_tl[4] = {__builtin_amdgcn_s_memrealtime(), 0ull, 0ull, 0ull};            \
    const unsigned gr_launch = timeline::g_count[blockIdx.x];
#define GEMM_RELU_MARK(point) gr_tl[point] = __builtin_amdgcn_s_memrealtime();
// Record: 5 stamps; where the workgroup ran: XCC_ID (hardware register 20) in
// bits 16 and up, and the low half of HW_ID (hardware register 4: CU in bits
// 8-11, shader array in bit 12, shader engine in bits 13-15); and the origin of
// the tile it computed last (the hooks expand inside gemm_relu_dma, whose
// c_m0 / c_n0 hold it), m0 in the high 32 bits.
#define GEMM_RELU_TIMELINE_END                                                                      \
    if (threadIdx.x == 0 && gr_launch < timeline::g_max_launches) {                                 \
        unsigned long long* gr_r = timeline::g_rec + ((size_t)gr_launch * gridDim.x + blockIdx.x) * 7; \
        gr_r[0] = gr_tl[0];                                                                         \
        gr_r[1] = gr_tl[1];                                                                         \
        gr_r[2] = gr_tl[2];                                                                         \
        gr_r[3] = gr_tl[3];                                                                         \
        gr_r[4] = __builtin_amdgcn_s_memrealtime();                                                 \
        gr_r[5] = ((unsigned long long)(__builtin_amdgcn_s_getreg(20 | (31 << 11)) & 0xffffu) << 16) |  \
                  (__builtin_amdgcn_s_getreg(4 | (31 << 11)) & 0xffffu);                            \
        gr_r[6] = ((unsigned long long)(unsigned)c_m0 << 32) | (unsigned)c_n0;                      \
        timeline::g_count[blockIdx.x] = gr_launch + 1;                                              \
    }

#include "gemm_relu_kernels.hpp"

namespace {

using namespace gemm_relu_hip;

#define CHECK(x)                                                                                    \
    do {                                                                                            \
        hipError_t e_ = (x);                                                                        \
        if (e_ != hipSuccess) {                                                                     \
            std::fprintf(stderr, "%s failed: %s (line %d)\n", #x, hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                                           \
        }                                                                                           \
    } while (0)

constexpr int kMaxLaunches = 256, kMaxGrid = 1024, kSets = 3, kWarm = 3, kRec = 7;

// splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014) and the Box-Muller transform.
struct Rng {
    uint64_t s;
    uint64_t next()
    {
        uint64_t z = (s += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    }
    double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }   // (0, 1)
};

uint16_t to_bits(float x, int dt)   // round to nearest, ties to even (finite x)
{
    if (dt == kF16) {
        const _Float16 h = (_Float16)x;
        uint16_t u;
        std::memcpy(&u, &h, 2);
        return u;
    }
    uint32_t u;
    std::memcpy(&u, &x, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

double from_bits(uint16_t u, int dt)
{
    if (dt == kF16) {
        _Float16 h;
        std::memcpy(&h, &u, 2);
        return (double)h;
    }
    const uint32_t w = (uint32_t)u << 16;
    float x;
    std::memcpy(&x, &w, 4);
    return (double)x;
}

void fill_normal(std::vector<uint16_t>& v, double sigma, uint64_t seed, int dt)
{
    Rng g{seed};
    for (size_t i = 0; i + 1 < v.size(); i += 2) {
        const double r = sigma * std::sqrt(-2.0 * std::log(g.uniform())), t = 6.283185307179586 * g.uniform();
        v[i] = to_bits((float)(r * std::cos(t)), dt);
        v[i + 1] = to_bits((float)(r * std::sin(t)), dt);
    }
}

double median(std::vector<double> v)
{
    std::sort(v.begin(), v.end());
    const size_t n = v.size();
    return n == 0 ? 0.0 : (n % 2 ? v[n / 2] : 0.5 * (v[n / 2 - 1] + v[n / 2]));
}

double quantile(std::vector<double> v, double q)   // nearest rank
{
    if (v.empty()) return 0.0;
    std::sort(v.begin(), v.end());
    const size_t i = (size_t)std::ceil(q * (double)v.size());
    return v[i == 0 ? 0 : i - 1];
}

struct Shape {
    const char* name;
    const char* config;
    int M, N, K, dt;
    double sigma;
};

// Runs one shape on gemm_relu_dma<Cfg, DT, 0>; returns the number of sampled mismatches.
template <class Cfg, int DT>
int run(const Shape& sh, int reps, int cus, double ticks_per_us)
{
    static_assert(DT == kF16 || DT == kBF16, "dtype");
    int M = sh.M, N = sh.N, K = sh.K;
    if (M % Cfg::BM || N % Cfg::BN || K % Cfg::BK) {
        std::fprintf(stderr, "%s: not whole tiles of the configuration\n", sh.name);
        std::exit(2);
    }
    int tiles_m = M / Cfg::BM, tiles_n = N / Cfg::BN, c_vec_ok = 2, splits = 1;
    const int grid = std::min(tiles_m * tiles_n, cus);
    if (grid > kMaxGrid || kWarm + reps > kMaxLaunches) {
        std::fprintf(stderr, "%s: grid or launch count beyond the record buffer\n", sh.name);
        std::exit(2);
    }
    std::vector<uint16_t> ha((size_t)M * K), hb((size_t)K * N);
    fill_normal(ha, sh.sigma, 1, DT);
    fill_normal(hb, sh.sigma, 2, DT);
    uint16_t *A[kSets], *B[kSets], *C[kSets];
    for (int s = 0; s < kSets; ++s) {
        CHECK(hipMalloc(&A[s], ha.size() * 2));
        CHECK(hipMalloc(&B[s], hb.size() * 2));
        CHECK(hipMalloc(&C[s], (size_t)M * N * 2));
        CHECK(hipMemcpy(A[s], ha.data(), ha.size() * 2, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(B[s], hb.data(), hb.size() * 2, hipMemcpyHostToDevice));
    }
    unsigned* count;
    unsigned long long* rec;
    CHECK(hipMalloc(&count, kMaxGrid * sizeof(unsigned)));
    CHECK(hipMalloc(&rec, (size_t)kMaxLaunches * kMaxGrid * kRec * sizeof(unsigned long long)));
    CHECK(hipMemset(count, 0, kMaxGrid * sizeof(unsigned)));
    CHECK(hipMemset(rec, 0, (size_t)kMaxLaunches * kMaxGrid * kRec * sizeof(unsigned long long)));
    const unsigned max_launches = kMaxLaunches;
    CHECK(hipMemcpyToSymbol(HIP_SYMBOL(timeline::g_count), &count, sizeof(count)));
    CHECK(hipMemcpyToSymbol(HIP_SYMBOL(timeline::g_rec), &rec, sizeof(rec)));
    CHECK(hipMemcpyToSymbol(HIP_SYMBOL(timeline::g_max_launches), &max_launches, sizeof(max_launches)));
    CHECK(hipDeviceSynchronize());

    float* ws = nullptr;
    int* counters = nullptr;
    auto launch = [&](int i) {
        const uint16_t *a = A[i % kSets], *b = B[i % kSets];
        uint16_t* c = C[i % kSets];
        void* args[] = {&a, &b, &c, &M, &N, &K, &tiles_m, &tiles_n, &c_vec_ok, &ws, &counters, &splits};
        CHECK(hipLaunchKernel((const void*)&gemm_relu_dma<Cfg, DT, 0>, dim3(grid), dim3(Cfg::THREADS), args, 0,
                              nullptr));
    };
    for (int i = 0; i < kWarm; ++i) launch(i);
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    CHECK(hipEventRecord(e0, nullptr));
    for (int i = 0; i < reps; ++i) launch(kWarm + i);
    CHECK(hipEventRecord(e1, nullptr));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));

    std::vector<unsigned> hcount(grid);
    std::vector<unsigned long long> hrec((size_t)kMaxLaunches * kMaxGrid * kRec);
    CHECK(hipMemcpy(hcount.data(), count, grid * sizeof(unsigned), hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(hrec.data(), rec, hrec.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
    for (int w = 0; w < grid; ++w)
        if (hcount[w] != (unsigned)(kWarm + reps)) {
            std::fprintf(stderr, "%s: workgroup %d recorded %u launches, expected %d\n", sh.name, w, hcount[w],
                         kWarm + reps);
            std::exit(1);
        }
    auto us = [&](unsigned long long a, unsigned long long b) { return (double)(long long)(b - a) / ticks_per_us; };
    std::vector<double> ramp, first, loop, epi, drain, span, gap;
    // Exit times (after the launch's first entry) of every workgroup of every launch, by
    // workgroup, and by the XCD the workgroup ran on.
    std::vector<double> exits, xcd_exits[8];
    std::vector<std::vector<double>> wg_exits(grid);
    std::vector<unsigned> place(grid);   // placement of each workgroup in the last launch
    std::vector<unsigned long long> tile(grid);   // and its last tile's origin (m0 << 32 | n0)
    for (int l = kWarm; l < kWarm + reps; ++l) {
        const unsigned long long* r = &hrec[(size_t)l * grid * kRec];
        unsigned long long t0 = ~0ull, t0_max = 0, t4 = 0;
        std::vector<double> f, lp, ep, dr;
        for (int w = 0; w < grid; ++w) {
            const unsigned long long* x = r + (size_t)w * kRec;
            t0 = std::min(t0, x[0]);
            t0_max = std::max(t0_max, x[0]);
            t4 = std::max(t4, x[4]);
            f.push_back(us(x[0], x[1]));
            lp.push_back(us(x[1], x[2]));
            ep.push_back(us(x[2], x[3]));
            dr.push_back(us(x[3], x[4]));
        }
        for (int w = 0; w < grid; ++w) {
            exits.push_back(us(t0, r[(size_t)w * kRec + 4]));
            place[w] = (unsigned)r[(size_t)w * kRec + 5];
            tile[w] = r[(size_t)w * kRec + 6];
            xcd_exits[(place[w] >> 16) & 7].push_back(exits.back());
            wg_exits[w].push_back(exits.back());
        }
        ramp.push_back(us(t0, t0_max));
        first.push_back(median(f));
        loop.push_back(median(lp));
        epi.push_back(median(ep));
        drain.push_back(median(dr));
        span.push_back(us(t0, t4));
        if (l + 1 < kWarm + reps) {
            const unsigned long long* n = &hrec[(size_t)(l + 1) * grid * kRec];
            unsigned long long n0 = ~0ull;
            for (int w = 0; w < grid; ++w) n0 = std::min(n0, n[(size_t)w * kRec]);
            gap.push_back(us(t4, n0));
        }
    }
    std::printf("{\"shape\": \"%s\", \"config\": \"%s\", \"M\": %d, \"N\": %d, \"K\": %d, \"dtype\": \"%s\", "
                "\"grid\": %d, \"units\": %d, \"launches\": %d, \"event_us\": %.2f, \"span_us\": %.2f, "
                "\"ramp_us\": %.2f, \"first_stage_us\": %.2f, \"k_loop_us\": %.2f, \"epilogue_us\": %.2f, "
                "\"store_drain_us\": %.2f, \"gap_us\": %.2f, \"exit_us\": {\"p10\": %.2f, \"p50\": %.2f, "
                "\"p90\": %.2f, \"max\": %.2f}, \"xcd_exit_p50_us\": [",
                sh.name, sh.config, M, N, K, DT == kF16 ? "fp16" : "bf16", grid, tiles_m * tiles_n, reps,
                ms * 1e3 / reps, median(span), median(ramp), median(first), median(loop), median(epi),
                median(drain), median(gap), quantile(exits, 0.1), quantile(exits, 0.5), quantile(exits, 0.9),
                quantile(exits, 1.0));
    for (int x = 0; x < 8; ++x) std::printf("%s%.2f", x ? ", " : "", median(xcd_exits[x]));
    // Per XCD, the shader engine whose workgroups' median exit is latest; and the workgroups whose
    // median exit over the launches is more than 15% after the median workgroup's, by placement.
    std::vector<double> wg_p50(grid);
    for (int w = 0; w < grid; ++w) wg_p50[w] = median(wg_exits[w]);
    const double typical = median(wg_p50);
    bool round_robin = true;   // workgroup w ran on XCD w % 8, as the tile remap assumes
    for (int w = 0; w < grid; ++w) round_robin = round_robin && ((place[w] >> 16) & 7) == (unsigned)(w % 8);
    std::printf("], \"xcd_is_wg_mod_8\": %s, \"slowest_se_per_xcd\": [", round_robin ? "true" : "false");
    for (int x = 0; x < 8; ++x) {
        int worst = -1;
        double worst_p50 = 0.0;
        for (int se = 0; se < 8; ++se) {
            std::vector<double> v;
            for (int w = 0; w < grid; ++w)
                if ((int)((place[w] >> 16) & 7) == x && (int)((place[w] >> 13) & 7) == se) v.push_back(wg_p50[w]);
            if (!v.empty() && median(v) > worst_p50) {
                worst_p50 = median(v);
                worst = se;
            }
        }
        std::printf("%s[%d, %.2f]", x ? ", " : "", worst, worst_p50);
    }
    std::printf("], \"slow_workgroups\": [");
    bool first_slow = true;
    for (int w = 0; w < grid; ++w)
        if (wg_p50[w] > 1.15 * typical) {
            // B stored (K, N): the tile's columns start at byte 2 n0 of every B row
            std::printf("%s{\"wg\": %d, \"xcd\": %u, \"se\": %u, \"cu\": %u, \"m0\": %u, \"n0\": %u, "
                        "\"b_row_byte\": %u, \"exit_p50_us\": %.2f}",
                        first_slow ? "" : ", ", w, (place[w] >> 16) & 7, (place[w] >> 13) & 7, (place[w] >> 8) & 15,
                        (unsigned)(tile[w] >> 32), (unsigned)tile[w], 2u * (unsigned)tile[w], wg_p50[w]);
            first_slow = false;
        }
    std::printf("]}\n");
    std::fflush(stdout);

    // C of the last launch (set (kWarm + reps - 1) % kSets) against fp64 sums on 64 sampled entries:
    // bf16 / fp16 rounding of C plus fp32 accumulation over K terms.
    std::vector<uint16_t> hc((size_t)M * N);
    CHECK(hipMemcpy(hc.data(), C[(kWarm + reps - 1) % kSets], hc.size() * 2, hipMemcpyDeviceToHost));
    const double rel = DT == kF16 ? 0x1p-10 : 0x1p-7;
    int bad = 0;
    for (int t = 0; t < 64; ++t) {
        const int m = (int)(((long long)t * 7919) % M), n = (int)(((long long)t * 104729 + 13) % N);
        double ref = 0.0, mag = 0.0;
        for (int k = 0; k < K; ++k) {
            const double p = from_bits(ha[(size_t)m * K + k], DT) * from_bits(hb[(size_t)k * N + n], DT);
            ref += p;
            mag += std::fabs(p);
        }
        ref = ref > 0.0 ? ref : 0.0;
        if (!(std::fabs(from_bits(hc[(size_t)m * N + n], DT) - ref) <= rel * ref + 1e-3 * mag)) ++bad;
    }
    if (bad) std::fprintf(stderr, "%s: %d of 64 sampled entries differ from fp64 sums\n", sh.name, bad);
    for (int s = 0; s < kSets; ++s) {
        CHECK(hipFree(A[s]));
        CHECK(hipFree(B[s]));
        CHECK(hipFree(C[s]));
    }
    CHECK(hipFree(count));
    CHECK(hipFree(rec));
    return bad;
}

}  // namespace

int main(int argc, char** argv)
{
    int reps = 20;
    std::string only;
    for (int i = 1; i < argc; ++i) {
        if (!std::strcmp(argv[i], "--reps") && i + 1 < argc) reps = std::atoi(argv[++i]);
        else if (!std::strcmp(argv[i], "--shape") && i + 1 < argc) only = argv[++i];
        else {
            std::fprintf(stderr, "usage: kernel_timeline [--reps N] [--shape NAME]\n");
            return 2;
        }
    }
    if (reps < 2 || kWarm + reps > kMaxLaunches) {
        std::fprintf(stderr, "reps in 2..%d\n", kMaxLaunches - kWarm);
        return 2;
    }
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    if (std::string(prop.gcnArchName).rfind("gfx950", 0) != 0) {
        std::fprintf(stderr, "needs a gfx950 GPU, found %s\n", prop.gcnArchName);
        return 2;
    }
    int rate_khz = 0;   // frequency of the s_memrealtime counter
    CHECK(hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, 0));
    if (rate_khz <= 0) {
        std::fprintf(stderr, "no wall-clock rate reported\n");
        return 1;
    }
    const double ticks_per_us = rate_khz / 1000.0;
    const int cus = prop.multiProcessorCount;
    const Shape shapes[] = {
        {"square_256", "8: 32x32x64, 4 stages, producer waves", 256, 256, 256, kF16, 1.0},
        {"square_1024", "9: 64x64x64, 4 stages, producer waves", 1024, 1024, 1024, kF16, 1.0},
        {"square_2048", "10: 128x128x64, 4 stages, producer waves", 2048, 2048, 2048, kF16, 1.0},
        {"skinny_64x16384x8192", "9: 64x64x64, 4 stages, producer waves", 64, 16384, 8192, kBF16, 0.05},
        {"square_8192", "3: 256x256x64, 2 stages, 16x16x32 MFMA, early refill", 8192, 8192, 8192, kF16, 0.1},
    };
    int bad = 0, ran = 0;
    for (const Shape& sh : shapes) {
        if (!only.empty() && only != sh.name) continue;
        ++ran;
        const std::string n = sh.name;
        if (n == "square_256") bad += run<DmaTile32W, kF16>(sh, reps, cus, ticks_per_us);
        else if (n == "square_1024") bad += run<DmaTile64W, kF16>(sh, reps, cus, ticks_per_us);
        else if (n == "square_2048") bad += run<DmaTile128W, kF16>(sh, reps, cus, ticks_per_us);
        else if (n == "skinny_64x16384x8192") bad += run<DmaTile64W, kBF16>(sh, reps, cus, ticks_per_us);
        else bad += run<DmaTile256, kF16>(sh, reps, cus, ticks_per_us);
    }
    if (ran == 0) {
        std::fprintf(stderr, "unknown shape %s\n", only.c_str());
        return 2;
    }
    std::printf("{\"checked\": %s, \"clock_mhz\": %.1f}\n", bad ? "false" : "true", ticks_per_us);
    return bad ? 1 : 0;
}
