// Power and shader clock of the two CDNA4 MFMA forms the kernels use, and of
// the 256 x 256 x 64 LDS-DMA tile built on each, on one MI355X.
//
// On normal fp16 data the 8192^3 GEMM runs at the board's power cap, where the
// shader clock, and with it the throughput, is set by the energy each flop
// costs.  This program measures that directly:
//
//   mode mfma: an MFMA-only loop, 8 waves per CU on all CUs, operands resident
//              in registers, once per shape (v_mfma_f32_32x32x16_f16 and
//              v_mfma_f32_16x16x32_f16, the same flops per iteration), on
//              N(0, 0.1^2) fp16 operands and on zeros;
//   mode tile: ReLU(A @ B) 8192^3 fp16 through the library's 256 tile
//              (gemm_relu_dma<DmaTile256>: 16x16x32, 128x64 waves, early
//              refill) and through the same tile on 32x32x16 MFMAs (64x128
//              waves, refill in the first k-step), three rotated input sets of
//              N(0, 0.1^2) entries.  First, both forms must give bit-identical
//              C on integer-valued inputs (every sum is exact in fp32), equal
//              to an fp64 host dot product on sampled entries.
//
// Each run launches back to back for --seconds while a host thread reads the
// shader clock (pp_dpm_sclk) and the package power (hwmon power1_average or
// power1_input) every 20 ms; the medians of the samples after the first
// third are reported.  Runs alternate between the two forms for --rounds.
//
// Usage: mfma_form [--mode mfma|tile|all] [--seconds S] [--rounds R]
// Output: one JSON line per run (and one for the tile check); exit status 1
// if the check fails.
#include <hip/hip_runtime.h>

#include <strings.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <string>
#include <thread>
#include <vector>

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

// ---------------------------------------------------------------- MFMA-only loops

constexpr int kLoopWaves = 8;   // per workgroup, one workgroup per CU

// One iteration is 2^20 flop per wave in both forms: 32 MFMAs of 32x32x16
// (4 k-blocks x 8 blocks) or 64 of 16x16x32 (2 k-blocks x 32 blocks), on
// operands loaded once.  The snake order over the blocks matches the kernels'.
__global__ __launch_bounds__(64 * kLoopWaves, 1) void mfma_loop32(const u32x4* __restrict__ src, float* __restrict__ out,
                                                                   int iters)
{
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * kLoopWaves + (threadIdx.x >> 6);
    u32x4 fa[4][4], fb[4][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[k][i] = src[(((w * 4 + k) * 6 + i) & 4095) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[k][j] = src[(((w * 4 + k) * 6 + 4 + j) & 4095) * 64 + lane];
    }
    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{0};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int bi = t / 2, bj = (bi & 1) ? 1 - t % 2 : t % 2;
                acc[bi][bj] = mfma_32x32x16<kF16>(fa[k][bi], fb[k][bj], acc[bi][bj]);
            }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) s += acc[i][j][0] + acc[i][j][15];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(64 * kLoopWaves, 1) void mfma_loop16(const u32x4* __restrict__ src, float* __restrict__ out,
                                                                   int iters)
{
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * kLoopWaves + (threadIdx.x >> 6);
    u32x4 fa[2][8], fb[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
        for (int i = 0; i < 8; ++i) fa[k][i] = src[(((w * 2 + k) * 12 + i) & 4095) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[k][j] = src[(((w * 2 + k) * 12 + 8 + j) & 4095) * 64 + lane];
    }
    floatx4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int t = 0; t < 32; ++t) {
                const int bi = t / 4, bj = (bi & 1) ? 3 - t % 4 : t % 4;
                acc[bi][bj] = mfma_16x16x32<kF16>(fa[k][bi], fb[k][bj], acc[bi][bj]);
            }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s += acc[i][j][0] + acc[i][j][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// ---------------------------------------------------------------- the two tile forms

using Tile16 = DmaTile256;                               // the library's
using Tile32 = DmaConfig<256, 256, 64, 2, 4, 2, 4>;      // 32x32x16, 64x128 waves, no early refill
static_assert(Tile16::MF == 16 && Tile32::MF == 32 && Tile16::LDS_BYTES == Tile32::LDS_BYTES,
              "the two forms of one tile");

template <class Cfg>
void launch_tile(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K, int cus)
{
    int tiles_m = M / Cfg::BM, tiles_n = N / Cfg::BN, c_vec_ok = 2, splits = 1;
    float* ws = nullptr;
    int* counters = nullptr;
    void* args[] = {&A, &B, &C, &M, &N, &K, &tiles_m, &tiles_n, &c_vec_ok, &ws, &counters, &splits};
    CHECK(hipLaunchKernel((const void*)&gemm_relu_dma<Cfg, kF16, 0>, dim3(std::min(tiles_m * tiles_n, cus)),
                          dim3(Cfg::THREADS), args, 0, nullptr));
}

// ---------------------------------------------------------------- host helpers

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
    void normal_pair(double& x, double& y)
    {
        const double r = std::sqrt(-2.0 * std::log(uniform())), t = 6.283185307179586 * uniform();
        x = r * std::cos(t);
        y = r * std::sin(t);
    }
};

void fill_normal(std::vector<_Float16>& v, double sigma, uint64_t seed)
{
    Rng g{seed};
    for (size_t i = 0; i + 1 < v.size(); i += 2) {
        double x, y;
        g.normal_pair(x, y);
        v[i] = (_Float16)(sigma * x);
        v[i + 1] = (_Float16)(sigma * y);
    }
}

void fill_integer(std::vector<_Float16>& v, uint64_t seed)
{
    Rng g{seed};
    for (auto& x : v) x = (_Float16)(double)((int)(g.next() % 5) - 2);
}

// The sysfs device directory of the measured GPU: among the AMD cards with a
// shader-clock table, the one whose device link points at the PCI address
// `pci_addr` ("dddd:bb:dd.f"), else the first of them; "" if there is none.
std::string gpu_sysfs_dir(const std::string& pci_addr)
{
    std::string first;
    for (int c = 0; c < 64; ++c) {
        const std::string d = "/sys/class/drm/card" + std::to_string(c) + "/device";
        std::ifstream v(d + "/vendor");
        std::string s;
        if (!(v >> s && s == "0x1002" && std::ifstream(d + "/pp_dpm_sclk").good())) continue;
        if (first.empty()) first = d;
        char real[PATH_MAX];
        if (!pci_addr.empty() && realpath(d.c_str(), real)) {
            const char* base = std::strrchr(real, '/');
            if (base && !strcasecmp(base + 1, pci_addr.c_str())) return d;
        }
    }
    return first;
}

int read_sclk_mhz(const std::string& dir)
{
    std::ifstream f(dir + "/pp_dpm_sclk");
    std::string line;
    while (std::getline(f, line))
        if (line.find('*') != std::string::npos) {
            const size_t colon = line.find(':');
            if (colon != std::string::npos) return std::atoi(line.c_str() + colon + 1);
        }
    return -1;
}

double read_power_w(const std::string& dir)
{
    for (const char* name : {"power1_average", "power1_input"})
        for (int h = 0; h < 16; ++h) {
            std::ifstream f(dir + "/hwmon/hwmon" + std::to_string(h) + "/" + name);
            long long uw;
            if (f >> uw) return uw / 1e6;
        }
    return -1.0;
}

struct Sustained {
    double seconds_gpu = 0, per_launch_ms = 0;
    long launches = 0;
    int sclk = -1;
    double power = -1;
};

// Launch back to back (in batches of `batch`) for `seconds`, timing with HIP
// events, while a host thread samples clock and power every 20 ms.
template <class F>
Sustained run_sustained(F launch, double seconds, int batch, const std::string& dir)
{
    for (int i = 0; i < batch; ++i) launch(i);
    CHECK(hipDeviceSynchronize());
    std::atomic<bool> stop{false};
    std::vector<int> clk;
    std::vector<double> pw;
    std::thread sampler([&]() {
        while (!stop) {
            if (!dir.empty()) {
                clk.push_back(read_sclk_mhz(dir));
                pw.push_back(read_power_w(dir));
            }
            std::this_thread::sleep_for(std::chrono::milliseconds(20));
        }
    });
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const auto t0 = std::chrono::steady_clock::now();
    long n = 0;
    CHECK(hipEventRecord(e0, nullptr));
    while (std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() < seconds) {
        for (int i = 0; i < batch; ++i) launch((int)(n + i));
        n += batch;
        CHECK(hipDeviceSynchronize());
    }
    CHECK(hipEventRecord(e1, nullptr));
    CHECK(hipEventSynchronize(e1));
    stop = true;
    sampler.join();
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    Sustained r;
    r.seconds_gpu = ms * 1e-3;
    r.launches = n;
    r.per_launch_ms = ms / n;
    const size_t skip = clk.size() / 3;
    std::vector<int> c(clk.begin() + skip, clk.end());
    std::vector<double> p(pw.begin() + skip, pw.end());
    if (!c.empty()) {
        std::sort(c.begin(), c.end());
        std::sort(p.begin(), p.end());
        r.sclk = c[c.size() / 2];
        r.power = p[p.size() / 2];
    }
    return r;
}

int mode_mfma(double seconds, int rounds, int cus, const std::string& dir)
{
    constexpr int kIters = 4000;   // about 3.5 ms per launch at full rate
    const double flop = (double)cus * kLoopWaves * kIters * (1 << 20);
    std::vector<_Float16> host(4096 * 64 * 8);
    fill_normal(host, 0.1, 1001);
    u32x4 *normal = nullptr, *zero = nullptr;
    float* out = nullptr;
    CHECK(hipMalloc(&normal, host.size() * 2));
    CHECK(hipMalloc(&zero, host.size() * 2));
    CHECK(hipMalloc(&out, (size_t)cus * 64 * kLoopWaves * sizeof(float)));
    CHECK(hipMemcpy(normal, host.data(), host.size() * 2, hipMemcpyHostToDevice));
    CHECK(hipMemset(zero, 0, host.size() * 2));
    for (const char* data : {"normal", "zero"})
        for (int r = 0; r < rounds; ++r)
            for (int form = 0; form < 2; ++form) {
                const u32x4* src = std::strcmp(data, "zero") ? normal : zero;
                auto launch = [&](int) {
                    if (form == 0) mfma_loop32<<<cus, 64 * kLoopWaves>>>(src, out, kIters);
                    else mfma_loop16<<<cus, 64 * kLoopWaves>>>(src, out, kIters);
                };
                const Sustained s = run_sustained(launch, seconds, 4, dir);
                std::printf("{\"mode\": \"mfma\", \"data\": \"%s\", \"shape\": \"%s\", \"round\": %d, \"tflops\": %.1f, "
                            "\"sclk_mhz\": %d, \"power_w\": %.0f, \"launches\": %ld}\n",
                            data, form == 0 ? "32x32x16" : "16x16x32", r, flop * s.launches / s.seconds_gpu / 1e12,
                            s.sclk, s.power, s.launches);
                std::fflush(stdout);
            }
    CHECK(hipFree(normal));
    CHECK(hipFree(zero));
    CHECK(hipFree(out));
    return 0;
}

int mode_tile(double seconds, int rounds, int cus, const std::string& dir)
{
    const int M = 8192, N = 8192, K = 8192;
    const size_t elems = (size_t)M * K;   // = K * N = M * N
    std::vector<_Float16> ha(elems), hb(elems);
    uint16_t *A[3], *B[3], *C[3];
    for (int i = 0; i < 3; ++i) {
        CHECK(hipMalloc(&A[i], elems * 2));
        CHECK(hipMalloc(&B[i], elems * 2));
        CHECK(hipMalloc(&C[i], elems * 2));
    }
    // 1. integer-valued inputs: both forms bit-identical and equal to the host's exact sums
    fill_integer(ha, 2001);
    fill_integer(hb, 2002);
    CHECK(hipMemcpy(A[0], ha.data(), elems * 2, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(B[0], hb.data(), elems * 2, hipMemcpyHostToDevice));
    launch_tile<Tile16>(A[0], B[0], C[0], M, N, K, cus);
    launch_tile<Tile32>(A[0], B[0], C[1], M, N, K, cus);
    CHECK(hipDeviceSynchronize());
    std::vector<uint16_t> c16(elems), c32(elems);
    CHECK(hipMemcpy(c16.data(), C[0], elems * 2, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(c32.data(), C[1], elems * 2, hipMemcpyDeviceToHost));
    const bool identical = c16 == c32;
    int mismatches = 0;
    Rng pick{3001};
    for (int s = 0; s < 2000; ++s) {
        const int m = (int)(pick.next() % M), n = (int)(pick.next() % N);
        double sum = 0.0;
        for (int k = 0; k < K; ++k) sum += (double)ha[(size_t)m * K + k] * (double)hb[(size_t)k * N + n];
        const _Float16 want = (_Float16)(sum > 0.0 ? sum : 0.0);
        if (c16[(size_t)m * N + n] != __builtin_bit_cast(uint16_t, want)) ++mismatches;
    }
    std::printf("{\"mode\": \"tile\", \"check\": {\"bit_identical\": %s, \"sampled\": 2000, \"sampled_mismatches\": %d}}\n",
                identical ? "true" : "false", mismatches);
    std::fflush(stdout);
    if (!identical || mismatches) return 1;
    // 2. N(0, 0.1^2) inputs, three rotated sets (402 MB each), alternating forms
    fill_normal(ha, 0.1, 2003);
    fill_normal(hb, 0.1, 2004);
    for (int i = 0; i < 3; ++i) {
        CHECK(hipMemcpy(A[i], ha.data(), elems * 2, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(B[i], hb.data(), elems * 2, hipMemcpyHostToDevice));
    }
    const double flop = 2.0 * M * N * K;
    for (int r = 0; r < rounds; ++r)
        for (int form = 0; form < 2; ++form) {
            auto launch = [&](int i) {
                if (form == 0) launch_tile<Tile16>(A[i % 3], B[i % 3], C[i % 3], M, N, K, cus);
                else launch_tile<Tile32>(A[i % 3], B[i % 3], C[i % 3], M, N, K, cus);
            };
            const Sustained s = run_sustained(launch, seconds, 10, dir);
            std::printf("{\"mode\": \"tile\", \"form\": \"%s\", \"round\": %d, \"ms\": %.4f, \"tflops\": %.1f, "
                        "\"sclk_mhz\": %d, \"power_w\": %.0f, \"launches\": %ld}\n",
                        form == 0 ? "16x16x32" : "32x32x16", r, s.per_launch_ms, flop / (s.per_launch_ms * 1e-3) / 1e12,
                        s.sclk, s.power, s.launches);
            std::fflush(stdout);
        }
    for (int i = 0; i < 3; ++i) {
        CHECK(hipFree(A[i]));
        CHECK(hipFree(B[i]));
        CHECK(hipFree(C[i]));
    }
    return 0;
}

}  // namespace

int main(int argc, char** argv)
{
    std::string mode = "all";
    double seconds = 2.0;
    int rounds = 2;
    for (int i = 1; i < argc; ++i) {
        if (i + 1 >= argc) {
            std::fprintf(stderr, "option %s needs a value\n", argv[i]);
            return 2;
        }
        if (!std::strcmp(argv[i], "--mode")) mode = argv[++i];
        else if (!std::strcmp(argv[i], "--seconds")) seconds = std::atof(argv[++i]);
        else if (!std::strcmp(argv[i], "--rounds")) rounds = std::atoi(argv[++i]);
        else {
            std::fprintf(stderr, "unknown option %s\n", argv[i]);
            return 2;
        }
    }
    if ((mode != "all" && mode != "mfma" && mode != "tile") || !(seconds > 0.0 && seconds <= 30.0) || rounds < 1 ||
        rounds > 10) {
        std::fprintf(stderr, "usage: mfma_form [--mode mfma|tile|all] [--seconds 0..30] [--rounds 1..10]\n");
        return 2;
    }
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    if (std::string(prop.gcnArchName).rfind("gfx950", 0) != 0) {
        std::fprintf(stderr, "needs a gfx950 GPU, found %s\n", prop.gcnArchName);
        return 2;
    }
    char bus[32] = {0};
    const std::string dir =
        gpu_sysfs_dir(hipDeviceGetPCIBusId(bus, (int)sizeof bus, 0) == hipSuccess ? std::string(bus) : std::string());
    if (dir.empty()) std::fprintf(stderr, "no sysfs clock/power files: sclk and power are reported as -1\n");
    const int cus = prop.multiProcessorCount;
    int rc = 0;
    if (mode != "tile") rc |= mode_mfma(seconds, rounds, cus, dir);
    if (mode != "mfma") rc |= mode_tile(seconds, rounds, cus, dir);
    return rc;
}
