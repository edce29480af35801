// Prefill product Y[t][i] = s[i] * sum_k X[t][k] Wc[i][k] for many tokens t.
//
// "The AQLM Quantization Algorithm, Explained", Figure 2 of the MCQ section:
// the matrix product runs on dequantized half-precision weights.  Each
// workgroup owns a BM-token x BN-row output tile.  Per k-step of 64 inputs it
// decodes the BN x 64 W tile into LDS as fp16, stages the matching BM x 64
// X tile next to it, and runs 16x16x32 fp16 matrix-core products with fp32
// accumulation; the row scale is applied once in the epilogue.
//
// Software pipeline (one barrier per k-step, LDS double-buffered):
//   top of step k : write the X chunks and decoded W groups of step k+1
//                   (already in registers) into the idle LDS buffer, then
//                   issue the global loads of step k+2;
//   body          : fragment reads and products of step k;
//   barrier.
// 2x8 codewords come from an LDS copy of the two codebooks (interleaved
// replicas); 1x16 codewords are gathered from the L2-resident codebook one
// step earlier than they are written, from codes loaded one step before that.
// Consecutive workgroups take consecutive token tiles of one W tile, so with
// 8 token tiles every XCD keeps one X tile in its L2.
//
// This is the general kernel (any in % 8 == 0, both schemes).  Both schemes
// with in % 64 == 0 take the role-split pipeline of gemm_pipe.hip instead.
#include "aqlm_device.h"
#include "aqlm_launch.h"

namespace aqlm {

template <int SCHEME, int BM, int BN, int WAVES_M, int WAVES_N, int REPL, int BK = 64, int MINB = 1>
struct GemmCfg {
    static constexpr int kBK = BK;                  // inputs per k-step
    static constexpr int kBKG = BK / kGroup;        // groups per k-step
    static constexpr int kLdsStride = BK + 8;       // fp16 per LDS row (+16 B: conflict-free 16 B reads)
    static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
    static constexpr int kWM = BM / WAVES_M;        // wave tile (tokens)
    static constexpr int kWN = BN / WAVES_N;        // wave tile (rows)
    static constexpr int kFM = kWM / 16;            // 16x16 blocks per wave
    static constexpr int kFN = kWN / 16;
    static constexpr int kXChunks = BM * kBKG / kThreads;   // 16-byte X chunks per thread
    static constexpr int kWGroups = BN * kBKG / kThreads;   // W groups per thread
    static constexpr int kXTile = BM * kLdsStride;
    static constexpr int kWTile = BN * kLdsStride;
    static constexpr int kCbSlots = SCHEME == kScheme2x8 ? 2 * kCodewords2x8 * REPL : 1;
    static constexpr size_t kLds = (size_t)2 * (kXTile + kWTile) * 2 + (size_t)kCbSlots * 16;
    static_assert(BM * kBKG % kThreads == 0 && BN * kBKG % kThreads == 0, "tile/threads mismatch");
    static_assert(kWGroups == 1 || kWGroups == 2 || kWGroups == 4 || kWGroups == 8, "W groups per thread");
    static_assert(kLds * MINB <= 163840, "LDS budget");
};

template <int SCHEME, int BM, int BN, int WAVES_M, int WAVES_N, int REPL, int BK, int MINB, bool PIPE>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, MINB) void gemm_kernel(
    const uint8_t* __restrict__ codes, const f16* __restrict__ codebooks,
    const f16* __restrict__ scales, const f16* __restrict__ x, f16* __restrict__ y,
    int out, int in, int T) {
    using C = GemmCfg<SCHEME, BM, BN, WAVES_M, WAVES_N, REPL, BK, MINB>;
    constexpr int kBKG = C::kBKG;
    constexpr int kLdsStride = C::kLdsStride;
    extern __shared__ u32x4 smem[];
    f16* xs = reinterpret_cast<f16*>(smem);                 // [2][kXTile]
    f16* ws = xs + 2 * C::kXTile;                            // [2][kWTile]
    u32x4* cb = reinterpret_cast<u32x4*>(ws + 2 * C::kWTile);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int G = in / kGroup;
    const int n_tt = (T + BM - 1) / BM;
    const int n0 = (int)(blockIdx.x / n_tt) * BN;   // first output row of the tile
    const int t0 = (int)(blockIdx.x % n_tt) * BM;   // first token of the tile
    const int n_k = (G + kBKG - 1) / kBKG;

    // W decode role: row wr of the tile, groups wg0 .. wg0 + kWGroups - 1 of each step.
    constexpr int kThrPerRow = kBKG / C::kWGroups;
    const int wr = tid / kThrPerRow;
    const int wg0 = (tid % kThrPerRow) * C::kWGroups;
    const int wrow = n0 + wr;
    const bool wrow_ok = wrow < out;
    const int rep = tid % REPL;

    if constexpr (SCHEME == kScheme2x8) {
        for (int j = tid; j < C::kCbSlots; j += C::kThreads) {
            const int km = j / REPL;
            cb[j] = load16(codebooks + (size_t)((km & 1) * kCodewords2x8 + (km >> 1)) * kGroup);
        }
    }

    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    // ---- stage helpers --------------------------------------------------
    auto load_x = [&](int ks, u32x4 (&xr)[C::kXChunks]) {
#pragma unroll
        for (int it = 0; it < C::kXChunks; ++it) {
            const int c = it * C::kThreads + tid;
            const int r = c / kBKG, gq = c % kBKG;
            const int tok = t0 + r, grp = ks * kBKG + gq;
            xr[it] = (tok < T && grp < G) ? load16(x + (size_t)tok * in + (size_t)grp * kGroup) : zero4;
        }
    };
    auto store_x = [&](int buf, const u32x4 (&xr)[C::kXChunks]) {
        f16* dst = xs + buf * C::kXTile;
#pragma unroll
        for (int it = 0; it < C::kXChunks; ++it) {
            const int c = it * C::kThreads + tid;
            const int r = c / kBKG, gq = c % kBKG;
            *reinterpret_cast<u32x4*>(dst + r * kLdsStride + gq * kGroup) = xr[it];
        }
    };
    // Codes of this thread's groups at step ks, one 16-bit code per entry.  The
    // loads are unconditional (indices clamped into the matrix) so that no
    // branch forces a wait on them; groups outside the matrix are masked when
    // they are decoded.
    const uint16_t* crow_c = reinterpret_cast<const uint16_t*>(codes) + (size_t)(wrow_ok ? wrow : out - 1) * G;
    auto load_codes = [&](int ks, uint32_t (&cv)[C::kWGroups]) {
        const int grp = ks * kBKG + wg0;
#pragma unroll
        for (int q = 0; q < C::kWGroups; ++q) cv[q] = crow_c[min(grp + q, G - 1)];
    };
    auto group_ok = [&](int ks, int q) { return wrow_ok && (ks * kBKG + wg0 + q < G); };
    // 1x16: gather the codewords (zero for groups outside the matrix).
    auto gather_w = [&](int ks, const uint32_t (&cv)[C::kWGroups], u32x4 (&wv)[C::kWGroups]) {
#pragma unroll
        for (int q = 0; q < C::kWGroups; ++q) {
            const u32x4 v = load16(codebooks + (size_t)cv[q] * kGroup);
            wv[q] = group_ok(ks, q) ? v : zero4;
        }
    };
    // 2x8: sum the two codewords from the LDS codebook copy.
    auto lookup_w = [&](int ks, const uint32_t (&cv)[C::kWGroups], u32x4 (&wv)[C::kWGroups]) {
#pragma unroll
        for (int q = 0; q < C::kWGroups; ++q) {
            const f16x8 c0 = as_f16x8(cb[(2 * (cv[q] & 0xff)) * REPL + rep]);
            const f16x8 c1 = as_f16x8(cb[(2 * (cv[q] >> 8) + 1) * REPL + rep]);
            wv[q] = group_ok(ks, q) ? as_u32x4(c0 + c1) : zero4;
        }
    };
    auto store_w = [&](int buf, const u32x4 (&wv)[C::kWGroups]) {
        f16* dst = ws + buf * C::kWTile + wr * kLdsStride + wg0 * kGroup;
#pragma unroll
        for (int q = 0; q < C::kWGroups; ++q) *reinterpret_cast<u32x4*>(dst + q * kGroup) = wv[q];
    };

    f32x4 acc[C::kFM][C::kFN];
#pragma unroll
    for (int i = 0; i < C::kFM; ++i)
#pragma unroll
        for (int j = 0; j < C::kFN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // All fragments of the step are read before the first product, and the
    // scheduler is not allowed to sink the reads next to their uses, so the
    // products never wait on LDS latency one pair at a time.
    auto mma_step = [&](int buf) {
        const f16* xsb = xs + buf * C::kXTile + (wm * C::kWM + (lane & 15)) * kLdsStride;
        const f16* wsb = ws + buf * C::kWTile + (wn * C::kWN + (lane & 15)) * kLdsStride;
        constexpr int KK = BK / 32;
        f16x8 a[KK][C::kFM], b[KK][C::kFN];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int kc = kk * 32 + 8 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < C::kFM; ++i) a[kk][i] = *reinterpret_cast<const f16x8*>(xsb + i * 16 * kLdsStride + kc);
#pragma unroll
            for (int j = 0; j < C::kFN; ++j) b[kk][j] = *reinterpret_cast<const f16x8*>(wsb + j * 16 * kLdsStride + kc);
        }
        if constexpr (PIPE) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int i = 0; i < C::kFM; ++i)
#pragma unroll
                for (int j = 0; j < C::kFN; ++j) acc[i][j] = mfma16x16x32(a[kk][i], b[kk][j], acc[i][j]);
    };

    // ---- prologue ---------------------------------------------------------
    u32x4 xr[C::kXChunks];
    u32x4 wv[C::kWGroups];
    uint32_t c1[C::kWGroups], c2[C::kWGroups];   // codes of steps k+1 and k+2 (1x16: k+2, k+3)
    load_codes(0, c1);
    load_x(0, xr);
    __syncthreads();   // codebook copy staged
    if constexpr (SCHEME == kScheme2x8) lookup_w(0, c1, wv); else gather_w(0, c1, wv);
    store_x(0, xr);
    store_w(0, wv);
    // step 1 in registers
    load_codes(1, c1);
    load_x(1, xr);
    if constexpr (SCHEME == kScheme1x16) {
        gather_w(1, c1, wv);
        load_codes(2, c2);
    }
    __syncthreads();

    // ---- main loop: steps 0 .. n_k-2 --------------------------------------
    for (int ks = 0; ks + 1 < n_k; ++ks) {
        const int nb = (ks + 1) & 1;
        if constexpr (SCHEME == kScheme2x8) {
            lookup_w(ks + 1, c1, wv);
            store_x(nb, xr);
            store_w(nb, wv);
            load_codes(ks + 2, c1);
            load_x(ks + 2, xr);
        } else {
            store_x(nb, xr);
            store_w(nb, wv);
            gather_w(ks + 2, c2, wv);
            load_codes(ks + 3, c2);
            load_x(ks + 2, xr);
        }
        mma_step(ks & 1);
        __syncthreads();
    }
    mma_step((n_k - 1) & 1);

    // ---- epilogue: lane holds D[4*(l/16)+r][l%16] of block (i, j) ------------
#pragma unroll
    for (int j = 0; j < C::kFN; ++j) {
        const int col = n0 + wn * C::kWN + j * 16 + (lane & 15);
        if (col >= out) continue;
        const float s = (float)scales[col];
#pragma unroll
        for (int i = 0; i < C::kFM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = t0 + wm * C::kWM + i * 16 + 4 * (lane >> 4) + r;
                if (tok < T) y[(size_t)tok * out + col] = (f16)(acc[i][j][r] * s);
            }
        }
    }
}

template <int SCHEME, int BM, int BN, int WAVES_M, int WAVES_N, int REPL, int BK = 64, int MINB = 1, bool PIPE = true>
hipError_t launch_gemm_t(const void* codes, const void* codebooks, const void* scales,
                         const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                         hipStream_t stream) {
    using C = GemmCfg<SCHEME, BM, BN, WAVES_M, WAVES_N, REPL, BK, MINB>;
    auto kern = gemm_kernel<SCHEME, BM, BN, WAVES_M, WAVES_N, REPL, BK, MINB, PIPE>;
    if (C::kLds > 65536) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::kLds);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)(((out + BN - 1) / BN) * ((batch + BM - 1) / BM)));
    hipLaunchKernelGGL(kern, grid, dim3(C::kThreads), C::kLds, stream, (const uint8_t*)codes,
                       (const f16*)codebooks, (const f16*)scales, (const f16*)x, (f16*)y,
                       (int)out, (int)in, (int)batch);
    return hipGetLastError();
}

hipError_t launch_gemm(int scheme, const void* codes, const void* codebooks, const void* scales,
                       const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                       hipStream_t stream) {
    if (scheme == kScheme2x8) {
        if (in % 64 == 0)
            return launch_gemm_pipe_2x8(codes, codebooks, scales, x, y, out, in, batch, stream);
        return launch_gemm_t<kScheme2x8, 256, 128, 4, 2, 2>(codes, codebooks, scales, x, y, out, in, batch, stream);
    }
    if (in % 64 == 0) return launch_gemm_pipe_1x16(codes, codebooks, scales, x, y, out, in, batch, stream);
    return launch_gemm_t<kScheme1x16, 256, 128, 4, 2, 1>(codes, codebooks, scales, x, y, out, in, batch, stream);
}

}  // namespace aqlm
