// Prefill product Y[t][i] = s[i] * sum_k X[t][k] Wc[i][k] for many tokens t.
//
// "The AQLM Quantization Algorithm, Explained", Figure 2 of the MCQ section:
// the matrix product runs on dequantized half-precision weights.  Here each
// workgroup decodes a BN x BK tile of W into LDS (fp16), stages the matching
// BM x BK tile of X next to it, and feeds both to 16x16x32 fp16 matrix-core
// products with fp32 accumulation; the row scale is applied once in the
// epilogue.  The 2x8 codebooks sit in LDS (replicated, as in the GEMV); 1x16
// codewords are gathered from L2.
#include "aqlm_device.h"
#include "aqlm_launch.h"

namespace aqlm {

constexpr int kBM = 128;        // tokens per workgroup tile
constexpr int kBN = 128;        // output rows per workgroup tile
constexpr int kBK = 64;         // inputs per k-step (8 groups)
constexpr int kBKG = kBK / kGroup;
constexpr int kLdsStride = kBK + 8;  // fp16 elements per LDS row (+16 B: conflict-free 16 B reads)
constexpr int kGemmThreads = 256;    // 4 waves, 2 x 2, each 64 x 64
constexpr int kGemmRepl = 4;

template <int SCHEME>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                            const f16* __restrict__ codebooks,
                                                            const f16* __restrict__ scales,
                                                            const f16* __restrict__ x,
                                                            f16* __restrict__ y,
                                                            int out, int in, int T) {
    constexpr int kCbSlots = (SCHEME == kScheme2x8) ? 2 * kCodewords2x8 * kGemmRepl : 1;
    __shared__ u32x4 cb_lds[kCbSlots];
    __shared__ __attribute__((aligned(16))) f16 xs[kBM * kLdsStride];
    __shared__ __attribute__((aligned(16))) f16 ws[kBN * kLdsStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int G = in / kGroup;
    // Tile order: consecutive workgroups share one W tile (output-row block).
    const int n_tt = (T + kBM - 1) / kBM;
    const int n0 = (int)(blockIdx.x / n_tt) * kBN;   // first output row of the tile
    const int t0 = (int)(blockIdx.x % n_tt) * kBM;   // first token of the tile

    if constexpr (SCHEME == kScheme2x8) {
        for (int i = tid; i < 2 * kCodewords2x8; i += kGemmThreads) {
            const u32x4 v = load16(codebooks + (size_t)i * kGroup);
            const int m = i / kCodewords2x8, k = i % kCodewords2x8;
#pragma unroll
            for (int r = 0; r < kGemmRepl; ++r) cb_lds[(2 * k + m) * kGemmRepl + r] = v;
        }
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    const int n_kstep = (G + kBKG - 1) / kBKG;
    for (int ks = 0; ks < n_kstep; ++ks) {
        const int gk0 = ks * kBKG;   // first group of this k-step
        __syncthreads();             // previous tiles consumed (and codebook staged)
        // X tile: kBM rows x 8 groups of 16 B; 4 loads per thread.
#pragma unroll
        for (int it = 0; it < (kBM * kBKG) / kGemmThreads; ++it) {
            const int idx = it * kGemmThreads + tid;
            const int r = idx / kBKG, gq = idx % kBKG;
            const int tok = t0 + r, grp = gk0 + gq;
            const u32x4 v = (tok < T && grp < G)
                                ? load16(x + (size_t)tok * in + (size_t)grp * kGroup) : zero4;
            *reinterpret_cast<u32x4*>(xs + r * kLdsStride + gq * kGroup) = v;
        }
        // W tile: kBN rows x 8 groups; each thread decodes 4 groups of one row.
        {
            const int r = tid >> 1;
            const int gq0 = (tid & 1) * 4;
            const int row = n0 + r;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int grp = gk0 + gq0 + q;
                u32x4 v = zero4;
                if (row < out && grp < G) {
                    const uint32_t code =
                        reinterpret_cast<const uint16_t*>(codes)[(size_t)row * G + grp];
                    if constexpr (SCHEME == kScheme2x8) {
                        const int rep = tid % kGemmRepl;
                        const f16x8 c0 = as_f16x8(cb_lds[(2 * (code & 0xff)) * kGemmRepl + rep]);
                        const f16x8 c1 = as_f16x8(cb_lds[(2 * (code >> 8) + 1) * kGemmRepl + rep]);
                        v = as_u32x4(c0 + c1);
                    } else {
                        v = load16(codebooks + (size_t)code * kGroup);
                    }
                }
                *reinterpret_cast<u32x4*>(ws + r * kLdsStride + (gq0 + q) * kGroup) = v;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kBK / 32; ++kk) {
            const int kc = kk * 32 + 8 * (lane >> 4);
            f16x8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const f16x8*>(xs + (wm * 64 + i * 16 + (lane & 15)) * kLdsStride + kc);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const f16x8*>(ws + (wn * 64 + j * 16 + (lane & 15)) * kLdsStride + kc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
        }
    }

    // Epilogue: lane holds D[4*(l/16)+r][l%16] of block (i, j): token rows, output columns.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (col >= out) continue;
        const float s = (float)scales[col];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = t0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
                if (tok < T) y[(size_t)tok * out + col] = (f16)(acc[i][j][r] * s);
            }
        }
    }
}

hipError_t launch_gemm(int scheme, const void* codes, const void* codebooks, const void* scales,
                       const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                       hipStream_t stream) {
    const dim3 grid((unsigned)(((out + kBN - 1) / kBN) * ((batch + kBM - 1) / kBM)));
    if (scheme == kScheme2x8)
        hipLaunchKernelGGL(gemm_kernel<kScheme2x8>, grid, dim3(kGemmThreads), 0, stream,
                           (const uint8_t*)codes, (const f16*)codebooks, (const f16*)scales,
                           (const f16*)x, (f16*)y, (int)out, (int)in, (int)batch);
    else
        hipLaunchKernelGGL(gemm_kernel<kScheme1x16>, grid, dim3(kGemmThreads), 0, stream,
                           (const uint8_t*)codes, (const f16*)codebooks, (const f16*)scales,
                           (const f16*)x, (f16*)y, (int)out, (int)in, (int)batch);
    return hipGetLastError();
}

}  // namespace aqlm
