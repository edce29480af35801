// Prefill product Y[t][i] = s[i] * sum_k X[t][k] Wc[i][k] for many tokens t.
//
// "The AQLM Quantization Algorithm, Explained", Figure 2 of the MCQ section:
// the matrix product runs on dequantized half-precision weights.  Each
// workgroup owns a 256-token x 128-row output tile.  Per k-step of 64 inputs
// it decodes the 128 x 64 W tile (1024 groups) into LDS as fp16, stages the
// matching 256 x 64 X tile next to it, and runs 16x16x32 fp16 matrix-core
// products with fp32 accumulation.  LDS is double-buffered: the global loads
// and the codebook lookups of step k+1 are in flight while step k's
// products run, so one barrier per step suffices.  The row scale is applied
// once in the epilogue.
//
// 2x8 codewords come from an LDS copy of the two codebooks (two interleaved
// replicas); 1x16 codewords are gathered from the L2-resident codebook.
// Consecutive workgroups take consecutive token tiles of one W tile, so with
// 8 token tiles every XCD keeps one X tile in its L2.
#include "aqlm_device.h"
#include "aqlm_launch.h"

namespace aqlm {

constexpr int kBM = 256;             // tokens per workgroup tile
constexpr int kBN = 128;             // output rows per workgroup tile
constexpr int kBK = 64;              // inputs per k-step
constexpr int kBKG = kBK / kGroup;   // groups per k-step (8)
constexpr int kLdsStride = kBK + 8;  // fp16 per LDS row (+16 B: conflict-free 16 B reads)
constexpr int kGemmThreads = 512;    // 8 waves: 4 along tokens x 2 along rows, 64 x 64 each
constexpr int kGemmRepl = 2;
constexpr int kXChunks = kBM * kBKG / kGemmThreads;   // 16-byte X chunks per thread (4)
constexpr int kWGroups = kBN * kBKG / kGemmThreads;   // W groups decoded per thread (2)
constexpr int kXTile = kBM * kLdsStride;              // fp16 elements
constexpr int kWTile = kBN * kLdsStride;

template <int SCHEME>
struct GemmLds {
    f16 xs[2][kXTile];
    f16 ws[2][kWTile];
    u32x4 cb[SCHEME == kScheme2x8 ? 2 * kCodewords2x8 * kGemmRepl : 1];
};

// Codes of this thread's kWGroups groups (row r, groups gq0, gq0+1) at k-step ks.
__device__ __forceinline__ uint32_t gemm_load_codes(const uint8_t* __restrict__ codes, int row,
                                                    int out, int grp, int G) {
    if (row >= out) return 0u;
    const uint16_t* c16 = reinterpret_cast<const uint16_t*>(codes) + (size_t)row * G;
    if ((G & 1) == 0 && grp + 1 < G) return *reinterpret_cast<const uint32_t*>(c16 + grp);
    uint32_t v = 0;
    if (grp < G) v = c16[grp];
    if (grp + 1 < G) v |= (uint32_t)c16[grp + 1] << 16;
    return v;
}

template <int SCHEME>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                            const f16* __restrict__ codebooks,
                                                            const f16* __restrict__ scales,
                                                            const f16* __restrict__ x,
                                                            f16* __restrict__ y,
                                                            int out, int in, int T) {
    __shared__ GemmLds<SCHEME> L;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int G = in / kGroup;
    const int n_tt = (T + kBM - 1) / kBM;
    const int n0 = (int)(blockIdx.x / n_tt) * kBN;   // first output row of the tile
    const int t0 = (int)(blockIdx.x % n_tt) * kBM;   // first token of the tile
    const int n_k = (G + kBKG - 1) / kBKG;

    // W decode role: row wr of the tile, groups wg0, wg0+1 of each k-step.
    const int wr = tid >> 2;
    const int wg0 = (tid & 3) * kWGroups;
    const int wrow = n0 + wr;
    const int rep = tid % kGemmRepl;

    if constexpr (SCHEME == kScheme2x8) {
        for (int j = tid; j < 2 * kCodewords2x8 * kGemmRepl; j += kGemmThreads) {
            const int km = j / kGemmRepl;
            L.cb[j] = load16(codebooks + (size_t)((km & 1) * kCodewords2x8 + (km >> 1)) * kGroup);
        }
    }

    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    auto load_x = [&](int ks, u32x4 (&xr)[kXChunks]) {
#pragma unroll
        for (int it = 0; it < kXChunks; ++it) {
            const int c = it * kGemmThreads + tid;
            const int r = c / kBKG, gq = c % kBKG;
            const int tok = t0 + r, grp = ks * kBKG + gq;
            xr[it] = (tok < T && grp < G) ? load16(x + (size_t)tok * in + (size_t)grp * kGroup) : zero4;
        }
    };
    auto store_x = [&](int buf, const u32x4 (&xr)[kXChunks]) {
#pragma unroll
        for (int it = 0; it < kXChunks; ++it) {
            const int c = it * kGemmThreads + tid;
            const int r = c / kBKG, gq = c % kBKG;
            *reinterpret_cast<u32x4*>(&L.xs[buf][r * kLdsStride + gq * kGroup]) = xr[it];
        }
    };
    // Decodes this thread's two groups of k-step ks (codes cv) into wr[].
    auto decode_w = [&](int ks, uint32_t cv, u32x4 (&wv)[kWGroups]) {
#pragma unroll
        for (int q = 0; q < kWGroups; ++q) {
            const uint32_t c = (cv >> (16 * q)) & 0xffff;
            const bool ok = (wrow < out) && (ks * kBKG + wg0 + q < G);
            if constexpr (SCHEME == kScheme2x8) {
                const f16x8 c0 = as_f16x8(L.cb[(2 * (c & 0xff)) * kGemmRepl + rep]);
                const f16x8 c1 = as_f16x8(L.cb[(2 * (c >> 8) + 1) * kGemmRepl + rep]);
                wv[q] = ok ? as_u32x4(c0 + c1) : zero4;
            } else {
                const u32x4 v = load16(codebooks + (size_t)c * kGroup);
                wv[q] = ok ? v : zero4;
            }
        }
    };
    auto store_w = [&](int buf, const u32x4 (&wv)[kWGroups]) {
#pragma unroll
        for (int q = 0; q < kWGroups; ++q)
            *reinterpret_cast<u32x4*>(&L.ws[buf][wr * kLdsStride + (wg0 + q) * kGroup]) = wv[q];
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Prologue: step 0 into buffer 0; codes of step 1 in flight.
    u32x4 xr[kXChunks];
    u32x4 wv[kWGroups];
    uint32_t c_next = gemm_load_codes(codes, wrow, out, 0 * kBKG + wg0, G);
    load_x(0, xr);
    uint32_t c_cur = c_next;
    c_next = (n_k > 1) ? gemm_load_codes(codes, wrow, out, 1 * kBKG + wg0, G) : 0u;
    __syncthreads();   // codebook staged
    decode_w(0, c_cur, wv);
    store_x(0, xr);
    store_w(0, wv);
    __syncthreads();

    for (int ks = 0; ks < n_k; ++ks) {
        const int buf = ks & 1;
        const bool more = ks + 1 < n_k;
        if (more) {
            load_x(ks + 1, xr);
            c_cur = c_next;
            c_next = (ks + 2 < n_k) ? gemm_load_codes(codes, wrow, out, (ks + 2) * kBKG + wg0, G) : 0u;
            if constexpr (SCHEME == kScheme1x16) decode_w(ks + 1, c_cur, wv);   // gathers in flight
        }
        const f16* xsb = L.xs[buf];
        const f16* wsb = L.ws[buf];
#pragma unroll
        for (int kk = 0; kk < kBK / 32; ++kk) {
            const int kc = kk * 32 + 8 * (lane >> 4);
            f16x8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const f16x8*>(xsb + (wm * 64 + i * 16 + (lane & 15)) * kLdsStride + kc);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const f16x8*>(wsb + (wn * 64 + j * 16 + (lane & 15)) * kLdsStride + kc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
        }
        if (more) {
            if constexpr (SCHEME == kScheme2x8) decode_w(ks + 1, c_cur, wv);
            store_x(buf ^ 1, xr);
            store_w(buf ^ 1, wv);
        }
        __syncthreads();
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
