// Kernels for any scheme: M codebooks (1..8) of 2^B codewords (B = 1..16) of
// g entries (g = 1, 2, 4, 8, 16 or 32).
//
// "The AQLM Quantization Algorithm, Explained", section "Key AQLM quantization
// parameters": (M, B, g) are free hyperparameters and many triples meet one bit
// budget, e.g. (1, 4), (2, 8), ..., (8, 32) at B = 8 for 2 bits; a B that is not
// a multiple of 8 leaves unused bits in the bytes that store a code.  So a code
// sits in whole bytes (uint8 for B <= 8, 16 bits for B <= 16) and its index is
// the low B bits.  Figure 2 of the MCQ section gives the dequantization: the M
// selected codewords are summed, then scaled by the row's factor.
//
// The 1x16 and 2x8 schemes at g = 8 have their own tuned kernels, and the GEMV
// of the other 2-bit B = 8 schemes (1x8 g4, 4x8 g16; 8x8 g32 above batch 8) runs
// the 2x8 one when in % 8 == 0; these serve every other case:
//   decode_generic_kernel : W16 exactly as the 1x16/2x8 decode kernel (fp32 sum
//                           from codebook 0 upward, fp32 scale, one RNE rounding),
//                           16-byte stores (for g < 8 and in % 8 == 0, 8/g
//                           groups a thread);
//   gemv_generic_kernel   : batch 1..16, one wave per row, 16 waves per
//                           workgroup, fp32 weights;
//   gemm_generic_kernel   : any batch, 128x128 tiles, W decoded into LDS in
//                           8-input chunks, 16x16x32 fp16 matrix-core products.
// g is a template parameter so that a group's g weights stay in registers; M
// and B are run-time values.  Codebooks of at most 64 KB are copied to LDS by
// the GEMM kernel and of at most 128 KB by the GEMV kernel (the 8x8 g=32 scheme's
// 128 KB included); larger ones are read through L2.
#include "aqlm_device.h"
#include "aqlm_launch.h"

namespace aqlm {

#pragma clang fp contract(off)

namespace {

constexpr size_t kGemvLdsCodebook = 131072;   // GEMV: bytes of codebook staged in LDS at most
constexpr size_t kGemmLdsCodebook = 65536;    // GEMM (next to its 40 KB of tiles)
constexpr int kGemvMaxBatchGeneric = 16;
constexpr int kGemvGenericThreads = 1024;     // 16 waves, one row each

// The codeword index of code i: the low B bits of its CB-byte stored pattern, or,
// for bit-packed codes (CB = 0), the B bits at bit i * B of the little-endian
// 32-bit word stream (least significant bit first; a code may straddle two words,
// and the second word is read only then).
template <int CB>
__device__ __forceinline__ uint32_t code_at(const uint8_t* __restrict__ codes, size_t i, uint32_t mask, int B) {
    if constexpr (CB == 1) {
        return (uint32_t)codes[i] & mask;
    } else if constexpr (CB == 2) {
        return (uint32_t)reinterpret_cast<const uint16_t*>(codes)[i] & mask;
    } else {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(codes);
        const uint64_t bit = (uint64_t)i * (uint64_t)B;
        const size_t wi = (size_t)(bit >> 5);
        const int off = (int)(bit & 31);
        uint32_t v = w[wi] >> off;
        if (off + B > 32) v |= w[wi + 1] << (32 - off);
        return v & mask;
    }
}

// N consecutive fp16 values starting at p (p aligned to 2N bytes, N <= 8).
template <int N>
__device__ __forceinline__ void load_f16(const f16* p, float (&v)[N]) {
    if constexpr (N == 8) {
        const f16x8 c = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = (float)c[t];
    } else if constexpr (N == 4) {
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        const f16x4 c = *reinterpret_cast<const f16x4*>(p);
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (float)c[t];
    } else if constexpr (N == 2) {
        const f16x2 c = *reinterpret_cast<const f16x2*>(p);
        v[0] = (float)c[0];
        v[1] = (float)c[1];
    } else {
        v[0] = (float)p[0];
    }
}

// Entries t0 .. t0+N-1 of the sum over m of the codewords selected by the M codes
// starting at codes[c0]: codebook 0's entry, then + codebook m, m ascending,
// each sum rounded to fp32.  cb points at codebook 0 ([M][2^B][G]).
template <int G, int N, int CB>
__device__ __forceinline__ void sum_codewords(const uint8_t* __restrict__ codes, size_t c0, const f16* cb,
                                              int M, int B, uint32_t mask, int t0, float (&v)[N]) {
    load_f16<N>(cb + (size_t)code_at<CB>(codes, c0, mask, B) * G + t0, v);
    for (int m = 1; m < M; ++m) {
        float c[N];
        load_f16<N>(cb + (((size_t)m << B) + code_at<CB>(codes, c0 + m, mask, B)) * G + t0, c);
#pragma unroll
        for (int t = 0; t < N; ++t) v[t] = __fadd_rn(v[t], c[t]);
    }
}

// The whole group (G entries) as fp32, in pieces of at most 8 entries.
template <int G, int CB>
__device__ __forceinline__ void group_weights(const uint8_t* __restrict__ codes, size_t c0, const f16* cb,
                                              int M, int B, uint32_t mask, float (&v)[G]) {
    constexpr int N = G < 8 ? G : 8;
#pragma unroll
    for (int p = 0; p < G / N; ++p) {
        float part[N];
        sum_codewords<G, N, CB>(codes, c0, cb, M, B, mask, p * N, part);
#pragma unroll
        for (int t = 0; t < N; ++t) v[p * N + t] = part[t];
    }
}

// Copies n_elems fp16 codebook entries into LDS: 16 bytes at a time when the
// size allows, else one entry at a time.
__device__ __forceinline__ void stage_codebook(f16* dst, const f16* __restrict__ src, size_t n_elems) {
    if ((n_elems & 7) == 0) {
        u32x4* d = reinterpret_cast<u32x4*>(dst);
        for (size_t i = threadIdx.x; i < n_elems / 8; i += blockDim.x) d[i] = load16(src + i * 8);
    } else {
        for (size_t i = threadIdx.x; i < n_elems; i += blockDim.x) dst[i] = src[i];
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Decode: one thread per KG consecutive groups, bit-exact.  KG = 1, or 8 / G for
// G < 8 when a row holds a whole number of 8-input pieces (in % 8 == 0): then the
// KG groups lie in one row and leave as one 16-byte store.  LDS: codebooks of at
// most kGemvLdsCodebook bytes are copied to LDS first (1024-thread workgroups),
// so the lookups are LDS reads instead of L2 gathers.
template <int G, int CB, bool LDS, int KG>
__global__ __launch_bounds__(1024) void decode_generic_kernel(const uint8_t* __restrict__ codes,
                                                              const f16* __restrict__ codebooks,
                                                              const f16* __restrict__ scales,
                                                              f16* __restrict__ w, uint32_t n_units,
                                                              uint32_t n_grp_row, int M, int B) {
    extern __shared__ u32x4 smem[];
    const f16* cb = codebooks;
    if constexpr (LDS) {
        f16* cbl = reinterpret_cast<f16*>(smem);
        stage_codebook(cbl, codebooks, (size_t)M << B << __builtin_ctz(G));
        cb = cbl;
    }
    const uint32_t mask = (1u << B) - 1u;
    // 64-bit loop index: n_units may come within a stride of 2^32 (see decode_kernel)
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t u64 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u64 < n_units; u64 += stride) {
        const uint32_t u = (uint32_t)u64;
        if constexpr (KG > 1) {
            static_assert(G * KG == 8, "one 16-byte store per unit");
            const uint32_t gid0 = u * KG;
            const float s = (float)scales[gid0 / n_grp_row];
            f16x8 o;
#pragma unroll
            for (int k = 0; k < KG; ++k) {
                float v[G];
                group_weights<G, CB>(codes, (size_t)(gid0 + k) * M, cb, M, B, mask, v);
#pragma unroll
                for (int t = 0; t < G; ++t) o[k * G + t] = (f16)__fmul_rn(v[t], s);
            }
            __builtin_nontemporal_store(o, reinterpret_cast<f16x8*>(w + (size_t)gid0 * G));
            continue;
        }
        const uint32_t gid = u;
        const float s = (float)scales[gid / n_grp_row];
        float v[G];
        group_weights<G, CB>(codes, (size_t)gid * M, cb, M, B, mask, v);
        f16* dst = w + (size_t)gid * G;
        if constexpr (G >= 8) {
#pragma unroll
            for (int p = 0; p < G / 8; ++p) {
                f16x8 o;
#pragma unroll
                for (int t = 0; t < 8; ++t) o[t] = (f16)__fmul_rn(v[p * 8 + t], s);
                // g <= 16: non-temporal, so the W16 stream does not evict the codebooks from L2;
                // g = 32: plain stores, which L2 merges into whole lines (a lane's four
                // 16-byte pieces are 64 bytes apart within one store instruction)
                if constexpr (G <= 16)
                    __builtin_nontemporal_store(o, reinterpret_cast<f16x8*>(dst + p * 8));
                else
                    *reinterpret_cast<f16x8*>(dst + p * 8) = o;
            }
        } else if constexpr (G > 1) {
            // one G-entry store per group: w is 16-byte aligned, so group gid starts at a
            // multiple of 2 G bytes; non-temporal, as above
            typedef _Float16 f16xg __attribute__((ext_vector_type(G)));
            f16xg o;
#pragma unroll
            for (int t = 0; t < G; ++t) o[t] = (f16)__fmul_rn(v[t], s);
            __builtin_nontemporal_store(o, reinterpret_cast<f16xg*>(dst));
        } else {
            dst[0] = (f16)__fmul_rn(v[0], s);
        }
    }
}

// ---------------------------------------------------------------------------
// GEMV, batch 1..16: wave w of a workgroup takes rows 16*blockIdx + w, stepping by
// 16*gridDim; lane l takes the row's groups l, l+64, ...  Weights stay fp32 (the
// scale is applied once per output); each lane accumulates its groups' dot
// products for every batch row, then the wave sums its lanes.
template <int G, int CB, bool LDS>
__global__ __launch_bounds__(kGemvGenericThreads) void gemv_generic_kernel(const uint8_t* __restrict__ codes,
                                                           const f16* __restrict__ codebooks,
                                                           const f16* __restrict__ scales,
                                                           const f16* __restrict__ x, f16* __restrict__ y,
                                                           int out, int in, int T, int M, int B) {
    extern __shared__ u32x4 smem[];
    const f16* cb = codebooks;
    if constexpr (LDS) {
        f16* cbl = reinterpret_cast<f16*>(smem);
        stage_codebook(cbl, codebooks, (size_t)M << B << __builtin_ctz(G));
        cb = cbl;
    }
    const uint32_t mask = (1u << B) - 1u;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_grp = in / G;
    constexpr int kRows = kGemvGenericThreads / 64;
    // 64-bit row index: out may come within a grid stride of 2^31
    for (int64_t row = (int64_t)blockIdx.x * kRows + wave; row < out; row += (int64_t)gridDim.x * kRows) {
        float acc[kGemvMaxBatchGeneric];
#pragma unroll
        for (int b = 0; b < kGemvMaxBatchGeneric; ++b) acc[b] = 0.f;
        for (int j = lane; j < n_grp; j += 64) {
            float v[G];
            group_weights<G, CB>(codes, ((size_t)row * n_grp + j) * M, cb, M, B, mask, v);
#pragma unroll
            for (int b = 0; b < kGemvMaxBatchGeneric; ++b) {
                if (b < T) {
                    constexpr int N = G < 8 ? G : 8;
                    float d = 0.f;
#pragma unroll
                    for (int p = 0; p < G / N; ++p) {
                        float xv[N];
                        load_f16<N>(x + (size_t)b * in + (size_t)j * G + p * N, xv);
#pragma unroll
                        for (int t = 0; t < N; ++t) d += v[p * N + t] * xv[t];
                    }
                    acc[b] += d;
                }
            }
        }
#pragma unroll
        for (int b = 0; b < kGemvMaxBatchGeneric; ++b) {
            if (b < T) {
                float a = acc[b];
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o, 64);
                acc[b] = a;
            }
        }
        if (lane == 0) {
            const float s = (float)scales[row];
#pragma unroll
            for (int b = 0; b < kGemvMaxBatchGeneric; ++b)
                if (b < T) y[(size_t)b * out + row] = (f16)(acc[b] * s);
        }
    }
}

// ---------------------------------------------------------------------------
// GEMM: a workgroup of 4 waves owns a 128-token x 128-row tile; k advances 32
// inputs per step.  Each thread decodes two 8-input chunks of W rows and loads
// two 16-byte chunks of X for the next step while the current one multiplies
// (LDS double-buffered, one barrier per step).  Rows past the end are clamped
// (their outputs are not written), inputs past the end are zero.
constexpr int kGBM = 128, kGBN = 128, kGBK = 32, kGStride = kGBK + 8;

template <int G, int CB, bool LDS>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const uint8_t* __restrict__ codes,
                                                           const f16* __restrict__ codebooks,
                                                           const f16* __restrict__ scales,
                                                           const f16* __restrict__ x, f16* __restrict__ y,
                                                           int out, int in, int T, int M, int B) {
    extern __shared__ u32x4 smem[];
    f16* xs = reinterpret_cast<f16*>(smem);          // [2][kGBM][kGStride]
    f16* ws = xs + 2 * kGBM * kGStride;              // [2][kGBN][kGStride]
    const f16* cb = codebooks;
    if constexpr (LDS) {
        f16* cbl = ws + 2 * kGBN * kGStride;
        stage_codebook(cbl, codebooks, (size_t)M << B << __builtin_ctz(G));
        cb = cbl;
    }
    const uint32_t mask = (1u << B) - 1u;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n_tt = (T + kGBM - 1) / kGBM;
    const int n0 = (int)(blockIdx.x / n_tt) * kGBN;
    const int t0 = (int)(blockIdx.x % n_tt) * kGBM;
    const int n_grp = in / G;
    const int n_k = (in + kGBK - 1) / kGBK;
    const bool x_vec = (in & 7) == 0;

    // 8 weights of row `row` starting at input k (k % 8 == 0); zero past the end
    auto decode_chunk = [&](int row, int k) -> f16x8 {
        float v[8];
        const size_t rbase = (size_t)row * n_grp;
        if constexpr (G >= 8) {
            if (k < in) {
                sum_codewords<G, 8, CB>(codes, (rbase + k / G) * M, cb, M, B, mask, k % G, v);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) v[t] = 0.f;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8 / G; ++q) {
                float part[G];
                const int kq = k + q * G;
                if (kq < in) {
                    sum_codewords<G, G, CB>(codes, (rbase + kq / G) * M, cb, M, B, mask, 0, part);
                } else {
#pragma unroll
                    for (int t = 0; t < G; ++t) part[t] = 0.f;
                }
#pragma unroll
                for (int t = 0; t < G; ++t) v[q * G + t] = part[t];
            }
        }
        f16x8 o;
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] = (f16)v[t];
        return o;
    };
    auto load_xchunk = [&](int tok, int k) -> f16x8 {
        const f16* p = x + (size_t)tok * in + k;
        if (x_vec && k + 8 <= in) return *reinterpret_cast<const f16x8*>(p);
        f16x8 o;
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] = (k + t < in) ? p[t] : (f16)0.f;
        return o;
    };
    // chunk c (0..511) of a tile: row c / 4, inputs 8 * (c % 4) .. + 8
    f16x8 xr[2], wr[2];
    auto fetch = [&](int ks) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int c = it * 256 + tid;
            const int r = c >> 2, k = ks * kGBK + 8 * (c & 3);
            xr[it] = load_xchunk(min(t0 + r, T - 1), k);
            wr[it] = decode_chunk(min(n0 + r, out - 1), k);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int c = it * 256 + tid;
            const int r = c >> 2, kc = 8 * (c & 3);
            *reinterpret_cast<f16x8*>(xs + (buf * kGBM + r) * kGStride + kc) = xr[it];
            *reinterpret_cast<f16x8*>(ws + (buf * kGBN + r) * kGStride + kc) = wr[it];
        }
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    fetch(0);
    store(0);
    __syncthreads();
    for (int ks = 0; ks < n_k; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < n_k) fetch(ks + 1);
        // lane l holds A[l%16][8(l/16)..] (tokens x k) and B[8(l/16)..][l%16] (k x rows)
        f16x8 a[4], b[4];
        const int kc = 8 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const f16x8*>(xs + (buf * kGBM + wm * 64 + i * 16 + (lane & 15)) * kGStride + kc);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = *reinterpret_cast<const f16x8*>(ws + (buf * kGBN + wn * 64 + j * 16 + (lane & 15)) * kGStride + kc);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
        if (ks + 1 < n_k) store(buf ^ 1);   // that buffer's last reader finished before the previous barrier
        __syncthreads();
    }
    // lane holds D[4*(l/16)+r][l%16] of block (i, j)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (col >= out) continue;
        const float s = (float)scales[col];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = t0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
                if (tok < T) y[(size_t)tok * out + col] = (f16)(acc[i][j][r] * s);
            }
    }
}

// ---------------------------------------------------------------------------
// Launch helpers: one instantiation per (g, code bytes[, codebook in LDS]).

size_t codebook_bytes(const GenericScheme& sc) { return ((size_t)sc.M << sc.B) * (size_t)sc.g * 2; }

template <int G, int CB, int KG>
hipError_t decode_gk(const GenericScheme& sc, const void* codes, const void* codebooks, const void* scales,
                     void* w, int64_t out, int64_t in, hipStream_t stream) {
    const uint32_t n_grp_row = (uint32_t)(in / G);
    const uint64_t n_units = (uint64_t)out * n_grp_row / KG;
    const size_t lds = codebook_bytes(sc);
    if (lds <= kGemvLdsCodebook) {   // codebooks in LDS: one or two 1024-thread workgroups per CU
        auto kern = decode_generic_kernel<G, CB, true, KG>;
        if (lds > 65536) {
            const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)lds);
            if (e != hipSuccess) return e;
        }
        uint64_t blocks = (n_units + 1023) / 1024;
        const uint64_t max_blocks = (uint64_t)device_cu_count() * (lds <= 65536 ? 2 : 1);
        if (blocks > max_blocks) blocks = max_blocks;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(1024), lds, stream, (const uint8_t*)codes,
                           (const f16*)codebooks, (const f16*)scales, (f16*)w, (uint32_t)n_units, n_grp_row, sc.M,
                           sc.B);
        return hipGetLastError();
    }
    uint64_t blocks = (n_units + 255) / 256;
    const uint64_t max_blocks = (uint64_t)device_cu_count() * 16;
    if (blocks > max_blocks) blocks = max_blocks;
    hipLaunchKernelGGL((decode_generic_kernel<G, CB, false, KG>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint8_t*)codes, (const f16*)codebooks, (const f16*)scales, (f16*)w,
                       (uint32_t)n_units, n_grp_row, sc.M, sc.B);
    return hipGetLastError();
}

template <int G, int CB>
hipError_t decode_g(const GenericScheme& sc, const void* codes, const void* codebooks, const void* scales,
                    void* w, int64_t out, int64_t in, hipStream_t stream) {
    if constexpr (G < 8) {
        if (in % 8 == 0) return decode_gk<G, CB, 8 / G>(sc, codes, codebooks, scales, w, out, in, stream);
    }
    return decode_gk<G, CB, 1>(sc, codes, codebooks, scales, w, out, in, stream);
}

template <int G, int CB, bool LDS>
hipError_t gemv_g(const GenericScheme& sc, const void* codes, const void* codebooks, const void* scales,
                  const void* x, void* y, int64_t out, int64_t in, int64_t batch, hipStream_t stream) {
    auto kern = gemv_generic_kernel<G, CB, LDS>;
    const size_t lds = LDS ? codebook_bytes(sc) : 0;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int64_t blocks_needed = (out + 15) / 16;
    const int64_t cap = (int64_t)device_cu_count() * (LDS ? 1 : 2);
    const int grid = (int)(blocks_needed < cap ? blocks_needed : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemvGenericThreads), lds, stream, (const uint8_t*)codes, (const f16*)codebooks,
                       (const f16*)scales, (const f16*)x, (f16*)y, (int)out, (int)in, (int)batch, sc.M, sc.B);
    return hipGetLastError();
}

template <int G, int CB, bool LDS>
hipError_t gemm_g(const GenericScheme& sc, const void* codes, const void* codebooks, const void* scales,
                  const void* x, void* y, int64_t out, int64_t in, int64_t batch, hipStream_t stream) {
    auto kern = gemm_generic_kernel<G, CB, LDS>;
    const size_t lds = (size_t)2 * (kGBM + kGBN) * kGStride * 2 + (LDS ? codebook_bytes(sc) : 0);
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)(((out + kGBN - 1) / kGBN) * ((batch + kGBM - 1) / kGBM)));
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, (const uint8_t*)codes, (const f16*)codebooks,
                       (const f16*)scales, (const f16*)x, (f16*)y, (int)out, (int)in, (int)batch, sc.M, sc.B);
    return hipGetLastError();
}

// Returns CALL(G, CB) for the scheme's g and code storage (CB = 1 byte for B <= 8,
// 2 bytes for B <= 16, 0 for bit-packed codes).
#define AQLM_CB(sc, G, CALL) (sc.packed ? CALL(G, 0) : (sc.B <= 8) ? CALL(G, 1) : CALL(G, 2))
#define AQLM_DISPATCH_G(sc, CALL)                                       \
    switch (sc.g) {                                                     \
        case 1: return AQLM_CB(sc, 1, CALL);                            \
        case 2: return AQLM_CB(sc, 2, CALL);                            \
        case 4: return AQLM_CB(sc, 4, CALL);                            \
        case 8: return AQLM_CB(sc, 8, CALL);                            \
        case 16: return AQLM_CB(sc, 16, CALL);                          \
        case 32: return AQLM_CB(sc, 32, CALL);                          \
        default: return hipErrorInvalidValue;                           \
    }

// Bit-packed codes from whole-byte ones: thread w builds 32-bit word w of the stream
// from the (at most 33) codes that overlap its bits [32 w, 32 w + 32).
template <int CB>
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes,
                                                         uint32_t* __restrict__ words, uint64_t n_codes,
                                                         uint64_t n_words, int B) {
    const uint32_t mask = (1u << B) - 1u;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; w < n_words; w += stride) {
        const uint64_t b0 = w * 32;
        const uint64_t n0 = b0 / (uint64_t)B;
        const uint64_t n1 = min(n_codes, (b0 + 32 + (uint64_t)B - 1) / (uint64_t)B);
        uint32_t acc = 0u;
        for (uint64_t n = n0; n < n1; ++n) {
            const uint32_t v = code_at<CB>(codes, (size_t)n, mask, B);
            const int64_t sh = (int64_t)(n * (uint64_t)B) - (int64_t)b0;   // -B < sh < 32
            acc |= sh < 0 ? v >> (int)(-sh) : v << (int)sh;
        }
        words[w] = acc;
    }
}

}  // namespace

uint64_t packed_code_words(int M, int B, int g, int64_t out, int64_t in) {
    const uint64_t n = (uint64_t)out * (uint64_t)(in / g) * (uint64_t)M;
    return (n * (uint64_t)B + 31) / 32;
}

hipError_t launch_pack_codes(const void* codes, void* words, int M, int B, int g, int64_t out, int64_t in,
                             hipStream_t stream) {
    const uint64_t n_codes = (uint64_t)out * (uint64_t)(in / g) * (uint64_t)M;
    const uint64_t n_words = packed_code_words(M, B, g, out, in);
    if (n_words == 0) return hipSuccess;
    uint64_t blocks = (n_words + 255) / 256;
    const uint64_t cap = (uint64_t)device_cu_count() * 16;
    if (blocks > cap) blocks = cap;
    if (B <= 8)
        hipLaunchKernelGGL(pack_codes_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint8_t*)codes, (uint32_t*)words, n_codes, n_words, B);
    else
        hipLaunchKernelGGL(pack_codes_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint8_t*)codes, (uint32_t*)words, n_codes, n_words, B);
    return hipGetLastError();
}

hipError_t launch_decode_generic(const GenericScheme& sc, const void* codes, const void* codebooks,
                                 const void* scales, void* w, int64_t out, int64_t in, hipStream_t stream) {
#define AQLM_DEC(G, CB) decode_g<G, CB>(sc, codes, codebooks, scales, w, out, in, stream)
    AQLM_DISPATCH_G(sc, AQLM_DEC)
#undef AQLM_DEC
}

hipError_t launch_gemv_generic(const GenericScheme& sc, const void* codes, const void* codebooks,
                               const void* scales, const void* x, void* y, int64_t out, int64_t in,
                               int64_t batch, hipStream_t stream) {
    const bool lds = codebook_bytes(sc) <= kGemvLdsCodebook;
#define AQLM_GV(G, CB) (lds ? gemv_g<G, CB, true>(sc, codes, codebooks, scales, x, y, out, in, batch, stream) \
                            : gemv_g<G, CB, false>(sc, codes, codebooks, scales, x, y, out, in, batch, stream))
    AQLM_DISPATCH_G(sc, AQLM_GV)
#undef AQLM_GV
}

hipError_t launch_gemm_generic(const GenericScheme& sc, const void* codes, const void* codebooks,
                               const void* scales, const void* x, void* y, int64_t out, int64_t in,
                               int64_t batch, hipStream_t stream) {
    const bool lds = codebook_bytes(sc) <= kGemmLdsCodebook;
#define AQLM_GM(G, CB) (lds ? gemm_g<G, CB, true>(sc, codes, codebooks, scales, x, y, out, in, batch, stream) \
                            : gemm_g<G, CB, false>(sc, codes, codebooks, scales, x, y, out, in, batch, stream))
    AQLM_DISPATCH_G(sc, AQLM_GM)
#undef AQLM_GM
}

}  // namespace aqlm
