// How fast the skinny decode-like GEMM's B can be streamed at all, beside the
// library's kernel for it.
//
// ReLU(A @ B) with M = 64, N = 16384, K = 8192 (bf16) is bound by reading B,
// 8192 rows of 32 KiB.  With one 64 x 64 tile per CU, each workgroup reads 128
// bytes of every row.  This program times, on 256 workgroups of 4 waves each
// filling LDS by direct-to-LDS loads (buffer_load_dwordx4 ... lds, 16 KiB per
// wave in flight) and doing nothing else, three read patterns over three
// rotated 256 MiB buffers:
//   contiguous  every DMA instruction reads 1 KiB of consecutive bytes;
//   strips      each workgroup reads its 128-byte column strip of every row,
//               64 rows per step, 8 rows per DMA instruction (the kernel's B
//               pattern);
//   strips_a    the same, with an 8 KiB step of a 1 MiB L2-resident buffer read
//               beside each B step (the kernel's A tiles);
//   strips_pitch_plus_128
//               the strips pattern over the same bytes laid out with a row
//               pitch of 32 KiB + 128 B: with the 32 KiB (power-of-two) pitch,
//               the 128-byte slot at byte 384 of every KiB of every row sits on
//               a narrower part of the memory system, and the workgroups that
//               read it set the pace;
// and then the library's kernels for the shape (the 64 x 64 tile with producer
// waves that its tuned table picks) on the same buffers, which hold N(0, 0.05^2)
// bf16 values as the workload's inputs do: with B stored (K, N), its 128-byte
// strips, and with B stored (N, K) (how decode weights are usually kept), where
// each workgroup reads 64 contiguous 16 KiB rows.  Each is
// launched back to back (--reps launches after 3 warm-up launches, three
// rotated buffer sets) and reported as B bytes per second.
//
// Usage: stream_ceiling [--reps N]
// Output: one JSON line per pattern, and per B layout one for the kernel and one
// for a sampled check of its C against fp64 sums (exit status 1 on a mismatch).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
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

constexpr int kRowBytes = 32768, kRows = 8192;           // B: 8192 rows of 16384 bf16
constexpr size_t kBBytes = (size_t)kRowBytes * kRows;    // 256 MiB
constexpr int kPaddedPitch = kRowBytes + 128;            // the padded layout's row pitch
constexpr size_t kBufBytes = (size_t)kPaddedPitch * kRows;   // room for either layout
constexpr int kARowBytes = 16384, kARows = 64;           // A: 64 rows of 8192 bf16 (1 MiB)
constexpr int kWaves = 4, kInFlight = 16;                // DMA instructions (1 KiB each) per wave in flight
constexpr int kGroups = 256;

// Slots of this wave's LDS ring: kInFlight KiB per wave.  After each full turn
// of the ring, wait until at most half of it is still in flight.
struct DmaRing {
    uint32_t base;
    int slot = 0;
    __device__ void issue(int32x4_t rsrc, uint32_t voff)
    {
        dma_b128(rsrc, base + slot * 1024, voff, 0u);
        if (++slot == kInFlight) {
            slot = 0;
            wait_vmcnt<kInFlight / 2>();
        }
    }
};

template <int MODE>   // 0 contiguous, 1 strips, 2 strips with the A stream, 3 strips at the padded pitch
__global__ __launch_bounds__(64 * kWaves) void stream_b(const uint8_t* __restrict__ b, const uint8_t* __restrict__ a,
                                                        unsigned* __restrict__ out)
{
    constexpr uint32_t pitch = MODE == 3 ? kPaddedPitch : kRowBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kWaves * kInFlight * 1024];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32x4_t rb = rsrc_words(b, (uint32_t)kBufBytes), ra = rsrc_words(a, kARowBytes * kARows);
    DmaRing ring{(uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem) + wave * kInFlight * 1024};
    if constexpr (MODE == 0) {
        // 1 KiB pieces: workgroup g, wave w takes pieces g*kWaves + w, + kGroups*kWaves, ...
        const uint32_t pieces = (uint32_t)(kBBytes / 1024);
        for (uint32_t p = blockIdx.x * kWaves + wave; p < pieces; p += gridDim.x * kWaves)
            ring.issue(rb, p * 1024u + lane * 16u);
    } else {
        // 8 rows x 128 bytes per instruction: lane l reads row 8 g + l / 8, bytes 16 (l % 8) of the strip
        const uint32_t col = blockIdx.x * 128u + (lane & 7) * 16u;
        for (int g = wave; g < kRows / 8; g += kWaves) {
            ring.issue(rb, (uint32_t)(g * 8 + (lane >> 3)) * pitch + col);
            if constexpr (MODE == 2) {
                // A: rows (g % 8) * 8 + l / 8 of 64, the 128-byte piece (g / 8) % 128 of each
                const uint32_t off = (uint32_t)((g & 7) * 8 + (lane >> 3)) * kARowBytes + ((g >> 3) & 127) * 128u +
                                     (lane & 7) * 16u;
                ring.issue(ra, off);
            }
        }
    }
    wait_vmcnt<0>();
    __syncthreads();
    if (smem[threadIdx.x] == 0xA5 && smem[threadIdx.x + 1] == 0x5A) out[0] = 1;   // keep the loads
}

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

uint16_t bf16_bits(float x)   // round to nearest, ties to even (finite x)
{
    uint32_t u;
    std::memcpy(&u, &x, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

void fill_normal_bf16(std::vector<uint16_t>& v, double sigma, uint64_t seed)
{
    Rng g{seed};
    for (size_t i = 0; i + 1 < v.size(); i += 2) {
        const double r = sigma * std::sqrt(-2.0 * std::log(g.uniform())), t = 6.283185307179586 * g.uniform();
        v[i] = bf16_bits((float)(r * std::cos(t)));
        v[i + 1] = bf16_bits((float)(r * std::sin(t)));
    }
}

// B bytes per second over `reps` back-to-back launches.
template <class F>
double rate(F launch, int reps)
{
    for (int i = 0; i < 3; ++i) launch(i);
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    CHECK(hipEventRecord(e0, nullptr));
    for (int i = 0; i < reps; ++i) launch(i);
    CHECK(hipEventRecord(e1, nullptr));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    return (double)kBBytes / (ms / reps * 1e-3);
}

constexpr int kM = 64, kN = 16384, kK = 8192;

struct Problem {
    const uint16_t* a;
    const uint16_t* b[3];
    uint16_t* c;
    const std::vector<uint16_t>* host_a;
    const std::vector<uint16_t>* host_b;   // kK x kN, or kN x kK when read as B stored (N, K)
    int cus;
};

double bf16_value(uint16_t h)
{
    const uint32_t u = (uint32_t)h << 16;
    float x;
    std::memcpy(&x, &u, 4);
    return (double)x;
}

// Times the library kernel gemm_relu_dma<Cfg> on the problem (B stored (N, K) if b_nk), then checks
// its C against fp64 sums on 256 sampled entries.  Allowed error: the bf16 rounding of C (2^-8
// relative) plus fp32 accumulation over K terms (1e-3 of the sum of |a b|).  Returns the number of
// mismatches.
template <class Cfg>
int run_kernel(const Problem& pr, bool b_nk, const char* name, int reps)
{
    static_assert(kM % Cfg::BM == 0 && kN % Cfg::BN == 0 && kK % Cfg::BK == 0, "whole tiles");
    int M = kM, N = kN, K = kK, tiles_m = kM / Cfg::BM, tiles_n = kN / Cfg::BN, c_vec_ok = 2, splits = 1;
    const int grid = std::min(tiles_m * tiles_n, pr.cus);
    float* ws = nullptr;
    int* counters = nullptr;
    auto launch = [&](int i) {
        const uint16_t *A = pr.a, *B = pr.b[i % 3];
        uint16_t* C = pr.c;
        void* args[] = {&A, &B, &C, &M, &N, &K, &tiles_m, &tiles_n, &c_vec_ok, &ws, &counters, &splits};
        CHECK(hipLaunchKernel((const void*)&gemm_relu_dma<Cfg, kBF16, 0>, dim3(grid), dim3(Cfg::THREADS), args, 0,
                              nullptr));
    };
    const char* layout = b_nk ? "nk" : "kn";
    std::printf("{\"kernel\": \"%s\", \"b_layout\": \"%s\", \"shape\": \"64x16384x8192 bf16\", "
                "\"workgroups\": %d, \"b_tbs\": %.3f}\n",
                name, layout, grid, rate(launch, reps) / 1e12);
    std::fflush(stdout);
    std::vector<uint16_t> hc((size_t)M * N);
    CHECK(hipMemcpy(hc.data(), pr.c, hc.size() * 2, hipMemcpyDeviceToHost));
    const auto &ha = *pr.host_a, &hb = *pr.host_b;
    int bad = 0;
    for (int t = 0; t < 256; ++t) {
        const int m = (t * 37) % M, n = (t * 4099 + 13) % N;
        double ref = 0.0, mag = 0.0;
        for (int k = 0; k < K; ++k) {
            const size_t bi = b_nk ? (size_t)n * K + k : (size_t)k * N + n;
            const double p = bf16_value(ha[(size_t)m * K + k]) * bf16_value(hb[bi]);
            ref += p;
            mag += std::fabs(p);
        }
        ref = ref > 0.0 ? ref : 0.0;
        if (!(std::fabs(bf16_value(hc[(size_t)m * N + n]) - ref) <= 0x1p-8 * ref + 1e-3 * mag)) ++bad;
    }
    std::printf("{\"check\": {\"b_layout\": \"%s\", \"sampled\": 256, \"mismatches\": %d}}\n", layout, bad);
    std::fflush(stdout);
    return bad;
}

}  // namespace

int main(int argc, char** argv)
{
    int reps = 50;
    for (int i = 1; i < argc; ++i) {
        if (!std::strcmp(argv[i], "--reps") && i + 1 < argc) reps = std::atoi(argv[++i]);
        else {
            std::fprintf(stderr, "usage: stream_ceiling [--reps N]\n");
            return 2;
        }
    }
    if (reps < 1 || reps > 10000) {
        std::fprintf(stderr, "reps in 1..10000\n");
        return 2;
    }
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    if (std::string(prop.gcnArchName).rfind("gfx950", 0) != 0) {
        std::fprintf(stderr, "needs a gfx950 GPU, found %s\n", prop.gcnArchName);
        return 2;
    }
    // Three rotated B buffers, one A buffer, one C buffer.
    uint8_t *b[3], *a;
    uint16_t* c;
    unsigned* flag;
    for (auto& p : b) CHECK(hipMalloc(&p, kBufBytes));
    CHECK(hipMalloc(&a, kARowBytes * kARows));
    CHECK(hipMalloc(&c, (size_t)64 * 16384 * 2));
    CHECK(hipMalloc(&flag, sizeof(unsigned)));
    // A and B ~ N(0, 0.05^2), rounded to bf16 (nearest, ties to even), as in the workload; the same B
    // in all three buffers.
    std::vector<uint16_t> host(kBBytes / 2), host_a((size_t)kARowBytes * kARows / 2);
    fill_normal_bf16(host, 0.05, 2);
    fill_normal_bf16(host_a, 0.05, 1);
    for (auto& p : b) CHECK(hipMemcpy(p, host.data(), kBBytes, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(a, host_a.data(), kARowBytes * kARows, hipMemcpyHostToDevice));
    const char* names[] = {"contiguous", "strips", "strips_a", "strips_pitch_plus_128"};
    for (int mode = 0; mode < 4; ++mode) {
        auto launch = [&](int i) {
            if (mode == 0) stream_b<0><<<kGroups, 64 * kWaves>>>(b[i % 3], a, flag);
            else if (mode == 1) stream_b<1><<<kGroups, 64 * kWaves>>>(b[i % 3], a, flag);
            else if (mode == 2) stream_b<2><<<kGroups, 64 * kWaves>>>(b[i % 3], a, flag);
            else stream_b<3><<<kGroups, 64 * kWaves>>>(b[i % 3], a, flag);
        };
        std::printf("{\"pattern\": \"%s\", \"workgroups\": %d, \"b_tbs\": %.3f}\n", names[mode], kGroups,
                    rate(launch, reps) / 1e12);
        std::fflush(stdout);
    }
    // The library's kernels for the shape, B stored (K, N) and (N, K) in the same buffers.
    Problem pr{reinterpret_cast<const uint16_t*>(a), {}, c, &host_a, &host, prop.multiProcessorCount};
    for (int i = 0; i < 3; ++i) pr.b[i] = reinterpret_cast<const uint16_t*>(b[i]);
    int bad = run_kernel<DmaTile64W>(pr, false, "gemm_relu_dma<DmaTile64W>", reps);
    bad += run_kernel<DmaTile64WT>(pr, true, "gemm_relu_dma<DmaTile64WT>", reps);
    for (auto& p : b) CHECK(hipFree(p));
    CHECK(hipFree(a));
    CHECK(hipFree(c));
    CHECK(hipFree(flag));
    return bad ? 1 : 0;
}
