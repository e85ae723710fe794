// Speed-of-light references: plain streaming kernels with the memory traffic
// of the hot path and none of its arithmetic.
//
//  k_sol_read        reads a buffer once with 16-byte non-temporal loads
//                    (the traffic of verification: every needed logit read
//                    once, nothing of size written back);
//  k_sol_read_write  reads two logit arrays and writes one fp32 array of the
//                    same length (the traffic of the VAT loss gradient:
//                    target and draft logits in, the gradient out).
//
// Both give one wavefront one 8 KiB slab per operand (64 lanes x 8 vectors of
// 16 bytes), all loads issued before the first use, in blocks of two
// wavefronts: the shape that read fastest in a sweep of block sizes (64 to
// 1024 threads), slabs per wavefront (1 to 4) and persistent grids on gfx950.
// The reductions only keep the loads alive: a result is stored only when the
// data hold a value the callers never put there.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kSolBlock = 128;
constexpr int kSolWaves = kSolBlock / kWave;
constexpr int kSolVec = kVecPerLane;                    // 16-byte vectors per lane per slab
constexpr int64_t kSolSlabVecs = int64_t{kWave} * kSolVec;  // 512 vectors = 8 KiB

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t nt_load(const u32x4_t* p) { return __builtin_nontemporal_load(p); }

__global__ __launch_bounds__(kSolBlock) void k_sol_read(const u32x4_t* data, int64_t nvec, uint32_t* sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t slab = static_cast<int64_t>(blockIdx.x) * kSolWaves + threadIdx.x / kWave;
    const u32x4_t* p = data + slab * kSolSlabVecs;
    const int64_t left = nvec - slab * kSolSlabVecs;
    u32x4_t v[kSolVec];
    if (left >= kSolSlabVecs) {
#pragma unroll
        for (int j = 0; j < kSolVec; ++j) v[j] = nt_load(p + j * kWave + lane);
    } else {
#pragma unroll
        for (int j = 0; j < kSolVec; ++j) {
            const int64_t i = j * kWave + lane;
            v[j] = i < left ? nt_load(p + i) : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < kSolVec; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    if (x == 0x9e3779b9u) sink[0] = x;  // keeps the loads; not reached by the benchmarks' data
}

// out[i] = a[i] - b[i] in fp32 (EB = 4: fp32 operands, 4 per vector; EB = 2:
// bf16 operands, 8 per vector, two output vectors per input vector).
template <int EB>
__global__ __launch_bounds__(kSolBlock) void k_sol_read_write(const u32x4_t* a, const u32x4_t* b, f32x4_t* out,
                                                              int64_t nvec) {
    constexpr int kOutPerIn = EB == 4 ? 1 : 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t slab = static_cast<int64_t>(blockIdx.x) * kSolWaves + threadIdx.x / kWave;
    const int64_t base = slab * kSolSlabVecs;
    const int64_t left = nvec - base;
    // a whole slab takes no per-vector tests, so its loads issue back to back
    const auto run = [&](auto whole) {
        constexpr bool kWhole = decltype(whole)::value;
        u32x4_t va[kSolVec], vb[kSolVec];
#pragma unroll
        for (int j = 0; j < kSolVec; ++j) {
            const int64_t i = j * kWave + lane;
            va[j] = kWhole || i < left ? nt_load(a + base + i) : u32x4_t{0u, 0u, 0u, 0u};
            vb[j] = kWhole || i < left ? nt_load(b + base + i) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kSolVec; ++j) {
            const int64_t i = j * kWave + lane;
            if (!kWhole && i >= left) continue;
            f32x4_t* o = out + (base + i) * kOutPerIn;
            if constexpr (EB == 4) {
                const f32x4_t r = {__uint_as_float(va[j].x) - __uint_as_float(vb[j].x),
                                   __uint_as_float(va[j].y) - __uint_as_float(vb[j].y),
                                   __uint_as_float(va[j].z) - __uint_as_float(vb[j].z),
                                   __uint_as_float(va[j].w) - __uint_as_float(vb[j].w)};
                __builtin_nontemporal_store(r, o);
            } else {
                const auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
                const auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
                const f32x4_t r0 = {lo(va[j].x) - lo(vb[j].x), hi(va[j].x) - hi(vb[j].x), lo(va[j].y) - lo(vb[j].y),
                                    hi(va[j].y) - hi(vb[j].y)};
                const f32x4_t r1 = {lo(va[j].z) - lo(vb[j].z), hi(va[j].z) - hi(vb[j].z), lo(va[j].w) - lo(vb[j].w),
                                    hi(va[j].w) - hi(vb[j].w)};
                __builtin_nontemporal_store(r0, o);
                __builtin_nontemporal_store(r1, o + 1);
            }
        }
    };
    if (left >= kSolSlabVecs)
        run(std::true_type{});
    else
        run(std::false_type{});
}

int64_t sol_blocks(int64_t nvec) {
    const int64_t slabs = (nvec + kSolSlabVecs - 1) / kSolSlabVecs;
    return (slabs + kSolWaves - 1) / kSolWaves;
}

}  // namespace

hipError_t launch_sol_read(const void* data, int64_t nvec, uint32_t* sink, hipStream_t stream) {
    if (nvec == 0) return hipSuccess;
    const int64_t blocks = sol_blocks(nvec);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_sol_read, dim3(static_cast<unsigned>(blocks)), dim3(kSolBlock), 0, stream,
                       static_cast<const u32x4_t*>(data), nvec, sink);
    return hipGetLastError();
}

hipError_t launch_sol_read_write(const void* a, const void* b, float* out, int64_t nvec, int elem_bytes,
                                 hipStream_t stream) {
    if (nvec == 0) return hipSuccess;
    const int64_t blocks = sol_blocks(nvec);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const auto* pa = static_cast<const u32x4_t*>(a);
    const auto* pb = static_cast<const u32x4_t*>(b);
    auto* po = reinterpret_cast<f32x4_t*>(out);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(k_sol_read_write<2>, dim3(static_cast<unsigned>(blocks)), dim3(kSolBlock), 0, stream, pa,
                           pb, po, nvec);
    else
        hipLaunchKernelGGL(k_sol_read_write<4>, dim3(static_cast<unsigned>(blocks)), dim3(kSolBlock), 0, stream, pa,
                           pb, po, nvec);
    return hipGetLastError();
}

}  // namespace sv
