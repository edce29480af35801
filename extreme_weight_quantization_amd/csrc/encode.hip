// Code assignment with fixed codebooks (greedy, residual) and residual k-means
// codebook initialisation.
//
// "The AQLM Quantization Algorithm, Explained", section "The AQLM quantization
// procedure": for each linear layer the codes are learned first, with the
// codebooks fixed and initialised by residual k-means.  The learning loss did
// not survive extraction and needs calibration data, so this is the
// data-free reading (the same one the CPU oracle states):
//
//   target of group n     r = W[i][j*g .. j*g+g) / s_i, one fp32 division each;
//   codebook m's code     the nearest codeword to r minus the codewords chosen
//                         for codebooks 0 .. m-1 (each subtraction in fp32),
//                         distance sum_t (r_t - c_t)^2 in fp32 with t ascending
//                         and no fused multiply-add, the lowest index on a tie;
//   residual k-means      Lloyd's algorithm on those leftovers for codebook 0,
//                         then 1, ...: seeds are given groups; a centroid is the
//                         mean of its members, summed exactly as integers in
//                         units of 2^-24 and divided in float64; an empty
//                         cluster keeps its centroid; the codebook is the fp16
//                         rounding of the centroids, and the codes are assigned
//                         against that fp16 codebook.
//
// Every integer decision (a code, a cluster label) therefore comes out of the
// same rounded operations as in the oracle, and the fixed-point sums make the
// centroids independent of the order of the atomic additions.
//
// The distance scan is a contraction (groups x codewords x g) but it stays on
// the vector ALUs: the matrix-core form |c|^2 - 2 r.c + |r|^2 rounds
// differently and would change which codeword is nearest.  One thread owns one
// group; the block streams the candidate codewords through LDS in 32 KB tiles,
// which all lanes read at the same address (a broadcast).
#include <algorithm>

#include "aqlm_device.h"
#include "aqlm_launch.h"

namespace aqlm {

#pragma clang fp contract(off)

namespace {

// One IEEE operation each, rounded to nearest-even, never fused with a neighbour.
// The runtime's rounded-operation intrinsics are plain operators in its own header,
// where contraction is allowed, so after inlining a product feeding a sum became a
// fused multiply-add (one rounding instead of two) and moved distance ties.  These
// are defined under this file's contract(off).
__device__ __forceinline__ float add_rn(float a, float b) { return a + b; }
__device__ __forceinline__ float sub_rn(float a, float b) { return a - b; }
__device__ __forceinline__ float mul_rn(float a, float b) { return a * b; }
__device__ __forceinline__ float div_rn(float a, float b) { return a / b; }

constexpr int kEncThreads = 256;
constexpr int kTileBytes = 32768;
constexpr double kFixedPoint = 16777216.0;          // 2^24
constexpr double kInvFixedPoint = 5.9604644775390625e-08;   // 2^-24
constexpr size_t kLdsAccBytes = 98304;                      // k-means sums kept in LDS up to this size

template <int CB>
__device__ __forceinline__ uint32_t load_code(const uint8_t* codes, size_t i, uint32_t mask) {
    if constexpr (CB == 1) return (uint32_t)codes[i] & mask;
    else return (uint32_t)reinterpret_cast<const uint16_t*>(codes)[i] & mask;
}

template <int CB>
__device__ __forceinline__ void store_code(uint8_t* codes, size_t i, uint32_t v) {
    if constexpr (CB == 1) codes[i] = (uint8_t)v;
    else reinterpret_cast<uint16_t*>(codes)[i] = (uint16_t)v;
}

// Leftover of group n after codebooks 0 .. m-1: W/s minus the chosen codewords.
template <int G, int CB>
__device__ __forceinline__ void residual(const f16* __restrict__ w, const f16* __restrict__ scales,
                                         const f16* __restrict__ codebooks, const uint8_t* __restrict__ codes,
                                         int64_t n, int64_t groups_per_row, int in, int M, int B, int m,
                                         float (&r)[G]) {
    const int64_t row = n / groups_per_row;
    const int64_t j = n - row * groups_per_row;
    const float s = (float)scales[row];
    const f16* src = w + row * in + j * G;
#pragma unroll
    for (int t = 0; t < G; ++t) r[t] = div_rn((float)src[t], s);
    const uint32_t mask = (1u << B) - 1u;
    for (int mm = 0; mm < m; ++mm) {
        const uint32_t k = load_code<CB>(codes, (size_t)n * M + mm, mask);
        const f16* c = codebooks + (((size_t)mm << B) + k) * G;
#pragma unroll
        for (int t = 0; t < G; ++t) r[t] = sub_rn(r[t], (float)c[t]);
    }
}

// Assignment of every group to its nearest candidate for codebook m.
//   FINAL  : candidates = fp16 codebook m; writes code m of the group.
//   KMEANS : candidates = fp32 centroids; adds the group's fixed-point leftover
//            to its cluster's sums and counts it.  With LACC the workgroup first
//            sums into LDS (dynamic shared memory, K*(G+1) int64) over all of its
//            groups and adds the non-zero totals to the global sums once at the
//            end: integer sums do not depend on the order, and the global
//            atomics drop from one per group to one per cluster and workgroup.
template <int G, int CB, bool KMEANS, bool LACC = false>
__global__ __launch_bounds__(kEncThreads) void assign_kernel(
    const f16* __restrict__ w, const f16* __restrict__ scales, const f16* __restrict__ codebooks,
    uint8_t* __restrict__ codes, const float* __restrict__ centroids, unsigned long long* __restrict__ sums,
    unsigned long long* __restrict__ counts, int64_t n_groups, int64_t groups_per_row, int in, int M, int B,
    int m, float lim = 0.f, unsigned long long* __restrict__ overflow = nullptr) {
    constexpr int kTile = kTileBytes / (4 * G);   // candidates per LDS tile
    __shared__ float tile[kTile * G];
    extern __shared__ unsigned long long lacc[];   // LACC: [K][G] sums, then [K] counts
    const int K = 1 << B;
    const f16* cbm = codebooks + ((size_t)m << B) * G;
    if constexpr (LACC) {
        for (int i = threadIdx.x; i < K * (G + 1); i += kEncThreads) lacc[i] = 0ull;
        __syncthreads();
    }
    for (int64_t base = (int64_t)blockIdx.x * kEncThreads; base < n_groups;
         base += (int64_t)gridDim.x * kEncThreads) {
        const int64_t n = base + threadIdx.x;
        const bool active = n < n_groups;
        float r[G];
        if (active) residual<G, CB>(w, scales, codebooks, codes, n, groups_per_row, in, M, B, m, r);
        float best = __builtin_inff();
        int best_k = 0;
        for (int k0 = 0; k0 < K; k0 += kTile) {
            const int nk = min(kTile, K - k0);
            __syncthreads();   // the previous tile has been read by every thread
            for (int i = threadIdx.x; i < nk * G; i += kEncThreads) {
                if constexpr (KMEANS) tile[i] = centroids[(size_t)k0 * G + i];
                else tile[i] = (float)cbm[(size_t)k0 * G + i];
            }
            __syncthreads();
            if (active) {
                for (int k = 0; k < nk; ++k) {
                    float d = 0.f;
#pragma unroll
                    for (int t = 0; t < G; ++t) {
                        const float e = sub_rn(r[t], tile[k * G + t]);
                        d = add_rn(d, mul_rn(e, e));
                    }
                    if (d < best) {
                        best = d;
                        best_k = k0 + k;
                    }
                }
            }
        }
        if (active) {
            if constexpr (KMEANS) {
                unsigned long long* ps = LACC ? lacc : sums;
                unsigned long long* pc = LACC ? lacc + (size_t)K * G : counts;
                // a target at or above lim (or not finite) could carry a cluster's sum out of
                // the exactly summed range: flag it, and the centroids come out NaN
                bool bad = false;
#pragma unroll
                for (int t = 0; t < G; ++t) bad |= !(__builtin_fabsf(r[t]) < lim);
                if (bad) atomicOr(overflow, 1ull);
#pragma unroll
                for (int t = 0; t < G; ++t) {
                    const long long q = bad ? 0ll : __double2ll_rn((double)r[t] * kFixedPoint);
                    atomicAdd(&ps[(size_t)best_k * G + t], (unsigned long long)q);
                }
                atomicAdd(&pc[best_k], 1ull);
            } else {
                store_code<CB>(codes, (size_t)n * M + m, (uint32_t)best_k);
            }
        }
    }
    if constexpr (LACC) {
        __syncthreads();
        for (int i = threadIdx.x; i < K * (G + 1); i += kEncThreads) {
            const unsigned long long v = lacc[i];
            if (v != 0ull) atomicAdd(i < K * G ? &sums[i] : &counts[i - K * G], v);
        }
    }
}

// Centroid k of codebook m starts as the leftover of group seeds[m][k] (clamped into range).
template <int G, int CB>
__global__ __launch_bounds__(kEncThreads) void seed_kernel(const f16* __restrict__ w, const f16* __restrict__ scales,
                                                          const f16* __restrict__ codebooks,
                                                          const uint8_t* __restrict__ codes,
                                                          const int64_t* __restrict__ seeds, float* __restrict__ centroids,
                                                          int64_t n_groups, int64_t groups_per_row, int in, int M,
                                                          int B, int m) {
    const int K = 1 << B;
    for (int k = blockIdx.x * kEncThreads + threadIdx.x; k < K; k += gridDim.x * kEncThreads) {
        int64_t n = seeds[(size_t)m * K + k];
        n = n < 0 ? 0 : (n >= n_groups ? n_groups - 1 : n);
        float r[G];
        residual<G, CB>(w, scales, codebooks, codes, n, groups_per_row, in, M, B, m, r);
#pragma unroll
        for (int t = 0; t < G; ++t) centroids[(size_t)k * G + t] = r[t];
    }
}

__global__ __launch_bounds__(kEncThreads) void zero_kernel(unsigned long long* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * kEncThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kEncThreads)
        p[i] = 0ull;
}

// Lloyd update: a non-empty cluster's centroid is its fixed-point sum / count (float64, then fp32).
// A flagged overflow makes every centroid NaN (and so every later codebook).
__global__ __launch_bounds__(kEncThreads) void update_kernel(const unsigned long long* __restrict__ sums,
                                                            const unsigned long long* __restrict__ counts,
                                                            float* __restrict__ centroids, int64_t n, int G,
                                                            const unsigned long long* __restrict__ overflow) {
    const bool bad = *overflow != 0ull;
    for (int64_t i = (int64_t)blockIdx.x * kEncThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kEncThreads) {
        if (bad) {
            centroids[i] = __builtin_nanf("");
            continue;
        }
        const unsigned long long c = counts[i / G];
        if (c == 0) continue;
        const double sum = (double)(long long)sums[i] * kInvFixedPoint;
        centroids[i] = __double2float_rn(__ddiv_rn(sum, (double)c));
    }
}

// Codebook m = fp16 rounding (nearest-even) of the centroids.
__global__ __launch_bounds__(kEncThreads) void round_kernel(const float* __restrict__ centroids,
                                                           f16* __restrict__ codebook, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * kEncThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kEncThreads)
        codebook[i] = (f16)centroids[i];
}

struct EncArgs {
    const f16* w;
    const f16* scales;
    f16* codebooks;
    uint8_t* codes;
    int64_t out, in;
    int M, B, g;
};

unsigned grid_for(int64_t items, int per_block_items) {
    const int64_t cap = (int64_t)device_cu_count() * 8;
    const int64_t need = (items + per_block_items - 1) / per_block_items;
    return (unsigned)(need < 1 ? 1 : (need < cap ? need : cap));
}

template <int G, int CB>
hipError_t assign_final(const EncArgs& a, int m, hipStream_t stream) {
    const int64_t gpr = a.in / G, n = a.out * gpr;
    hipLaunchKernelGGL((assign_kernel<G, CB, false>), dim3(grid_for(n, kEncThreads)), dim3(kEncThreads), 0, stream,
                       a.w, a.scales, a.codebooks, a.codes, nullptr, nullptr, nullptr, n, gpr, (int)a.in, a.M, a.B, m);
    return hipGetLastError();
}

template <int G, int CB>
hipError_t encode_g(const EncArgs& a, hipStream_t stream) {
    for (int m = 0; m < a.M; ++m) {
        const hipError_t e = assign_final<G, CB>(a, m, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int G, int CB>
hipError_t kmeans_g(const EncArgs& a, const int64_t* seeds, void* workspace, int iters, hipStream_t stream) {
    const int K = 1 << a.B;
    const int64_t gpr = a.in / G, n = a.out * gpr;
    unsigned long long* sums = static_cast<unsigned long long*>(workspace);
    unsigned long long* counts = sums + (size_t)K * G;
    float* centroids = reinterpret_cast<float*>(counts + K);
    // the flag sits after the centroids, 8-byte aligned (K G floats, K = 2^B >= 2)
    unsigned long long* overflow = reinterpret_cast<unsigned long long*>(centroids + (size_t)K * G);
    // targets below lim keep every coordinate sum over the n groups below 2^29 in magnitude,
    // i.e. below 2^53 grid units: exact as int64 and in its float64 conversion
    const float lim = (float)(536870912.0 / (double)(n > 0 ? n : 1));
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(kEncThreads), 0, stream, overflow, (int64_t)1);
    for (int m = 0; m < a.M; ++m) {
        hipLaunchKernelGGL((seed_kernel<G, CB>), dim3(grid_for(K, kEncThreads)), dim3(kEncThreads), 0, stream,
                           a.w, a.scales, a.codebooks, a.codes, seeds, centroids, n, gpr, (int)a.in, a.M, a.B, m);
        for (int it = 0; it < iters; ++it) {
            hipLaunchKernelGGL(zero_kernel, dim3(grid_for((int64_t)K * (G + 1), kEncThreads)), dim3(kEncThreads), 0,
                               stream, sums, (int64_t)K * (G + 1));
            const size_t lacc_bytes = (size_t)K * (G + 1) * 8;
            if (lacc_bytes <= kLdsAccBytes) {
                // as many workgroups per compute unit as LDS holds (at most 4), each summing many groups in LDS
                auto kern = assign_kernel<G, CB, true, true>;
                if (lacc_bytes > 32768) {
                    const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                                             (int)lacc_bytes);
                    if (e != hipSuccess) return e;
                }
                const int64_t need = (n + kEncThreads - 1) / kEncThreads;
                const int64_t per_cu = std::min<int64_t>(4, std::max<int64_t>(1, 163840 / (kTileBytes + (int64_t)lacc_bytes)));
                const int64_t cap = device_cu_count() * per_cu;
                hipLaunchKernelGGL(kern, dim3((unsigned)(need < cap ? need : cap)), dim3(kEncThreads), lacc_bytes,
                                   stream, a.w, a.scales, a.codebooks, a.codes, centroids, sums, counts, n, gpr,
                                   (int)a.in, a.M, a.B, m, lim, overflow);
            } else {
                hipLaunchKernelGGL((assign_kernel<G, CB, true>), dim3(grid_for(n, kEncThreads)), dim3(kEncThreads),
                                   0, stream, a.w, a.scales, a.codebooks, a.codes, centroids, sums, counts, n, gpr,
                                   (int)a.in, a.M, a.B, m, lim, overflow);
            }
            hipLaunchKernelGGL(update_kernel, dim3(grid_for((int64_t)K * G, kEncThreads)), dim3(kEncThreads), 0, stream,
                               sums, counts, centroids, (int64_t)K * G, G, overflow);
        }
        hipLaunchKernelGGL(round_kernel, dim3(grid_for((int64_t)K * G, kEncThreads)), dim3(kEncThreads), 0, stream,
                           centroids, a.codebooks + ((size_t)m << a.B) * G, (int64_t)K * G);
        const hipError_t e = assign_final<G, CB>(a, m, stream);
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}

#define AQLM_ENC_DISPATCH(g, B, CALL)                                   \
    switch (g) {                                                        \
        case 1: return (B <= 8) ? CALL(1, 1) : CALL(1, 2);              \
        case 2: return (B <= 8) ? CALL(2, 1) : CALL(2, 2);              \
        case 4: return (B <= 8) ? CALL(4, 1) : CALL(4, 2);              \
        case 8: return (B <= 8) ? CALL(8, 1) : CALL(8, 2);              \
        case 16: return (B <= 8) ? CALL(16, 1) : CALL(16, 2);           \
        case 32: return (B <= 8) ? CALL(32, 1) : CALL(32, 2);           \
        default: return hipErrorInvalidValue;                           \
    }

}  // namespace

int64_t kmeans_workspace_bytes(int M, int B, int g) {
    (void)M;
    const int64_t K = (int64_t)1 << B;
    return K * g * 8 + K * 8 + K * g * 4 + 16;   // fixed-point sums, counts, fp32 centroids, overflow flag
}

hipError_t launch_encode_greedy(const void* w, const void* scales, const void* codebooks, void* codes, int M, int B,
                                int g, int64_t out, int64_t in, hipStream_t stream) {
    const EncArgs a{(const f16*)w, (const f16*)scales, (f16*)codebooks, (uint8_t*)codes, out, in, M, B, g};
#define AQLM_ENC(G, CB) encode_g<G, CB>(a, stream)
    AQLM_ENC_DISPATCH(g, B, AQLM_ENC)
#undef AQLM_ENC
}

hipError_t launch_kmeans_init(const void* w, const void* scales, const int64_t* seeds, void* codebooks, void* codes,
                              void* workspace, int M, int B, int g, int64_t out, int64_t in, int iters,
                              hipStream_t stream) {
    const EncArgs a{(const f16*)w, (const f16*)scales, (f16*)codebooks, (uint8_t*)codes, out, in, M, B, g};
#define AQLM_KM(G, CB) kmeans_g<G, CB>(a, seeds, workspace, iters, stream)
    AQLM_ENC_DISPATCH(g, B, AQLM_KM)
#undef AQLM_KM
}

}  // namespace aqlm
