// Decode-phase product of the 2x8 scheme at batch 1-4 on large layers:
// y[b][i] = s[i] * sum_k Wc[i][k] x[b][k].
//
// "The AQLM Quantization Algorithm, Explained", section "Why and what do we
// quantize?" (decoding is memory-bound: the codes should stream at HBM rate)
// and section "What is Multi-Codebook Quantization (MCQ)?", Figure 2 (a group
// decodes to the sum of one codeword per codebook, times the row scale).
// Arithmetic: each codeword times x on the fp16 matrix cores with fp32
// accumulation (the two codewords of a group are two products, so their sum is
// never rounded to fp16), the scale applied once in fp32, one rounding of y.
// The schedule is built so that the only global loads in flight during the
// product are the codes, read in the order that streams best:
//
//  * one workgroup of 16 waves per CU owns the row tiles (16 rows) bid,
//    bid + nwg, ... of its layer, R of them;
//  * before the product the workgroup copies into LDS the codebooks (8
//    replicas, 64 KB) and all of x (T rows of in fp16), so activations are
//    LDS reads, not global loads; only the lanes of the T batch columns read x;
//  * the input is cut into slabs of 32 groups (64 bytes of codes a row); wave w
//    takes a contiguous range of the slabs (min(16, slabs) ranges) and walks
//    its tiles one after another, each over its whole range, so the two halves
//    of a row's 128-byte line are read back to back by the same wave;
//  * the codes of the next 2 steps are in flight in a ring of registers whose
//    slots are fixed at compile time, refilled unconditionally after their last
//    use, so the compiler waits for the oldest load only (two steps a wave, 2 KB,
//    stream faster than three or four: with 16 waves a CU the deeper rings
//    queue more requests than HBM serves well);
//  * a step issues its 16 codebook reads before its first product, and the
//    kernels are compiled for at most 4 waves a SIMD (one workgroup a CU), so
//    the registers for all 16 codewords are there;
//  * each wave writes one fp32 partial per (tile, row, batch column) to LDS at
//    the end of its range of a tile; after the last tile one barrier, and the
//    partials of a tile are added in slab-range order, scaled and rounded.  A
//    ragged last slab (in % 256 != 0) is added apart, masked, as one more
//    partial.
// The two codebook reads of a group go to distinct 16-byte bank groups for the
// 16 lanes served together (lane l reads codebook (l / 8) % 2 first), and an
// address is one v_perm_b32.  Results are deterministic, and a launch over
// several layers gives bit for bit what one launch per layer gives.
#include <algorithm>

#include "aqlm_device.h"
#include "aqlm_launch.h"

namespace aqlm {

namespace {

constexpr int kSWaves = 16;
constexpr int kSThreads = kSWaves * kWave;
constexpr int kSSlab = 32;                                  // groups per slab
constexpr int kSRepl = 8;                                   // codebook replicas
constexpr int kSCbBytes = 2 * kCodewords2x8 * kSRepl * 16;   // 64 KB
constexpr int kSRing = 2;                                   // steps of codes in flight per wave
constexpr int kSMaxT = 4;
constexpr int kSMinSteps = 2;                               // slab steps per wave below which gemv_kernel serves
constexpr int kSMinSteps34 = 4;                             // the same at batch 3-4 (x takes longer to stage)

// LDS read of 16 bytes at a byte address of the workgroup's LDS.  The kernels
// of this file declare no static LDS, so their dynamic LDS starts at address 0.
__device__ __forceinline__ u32x4 lds16(uint32_t byte) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((uintptr_t)byte);
}

// The 16 products of one chunk (a lane's 16 bytes of codes: groups 8 kq .. 8 kq + 7
// of its row in the slab, two codewords each) added to acc.  Codeword k of codebook m, replica r is
// at LDS byte 256 k + 128 m + 16 r; lane l uses replica l % 8 and reads codebook
// mA = (l / 8) % 2 first.  base: byte 0 = 16 r + 128 mA, byte 1 = 16 r + 128 (1 - mA).
// All 16 reads are issued before the first product.  MASKED: pieces whose ok bit
// is clear contribute zero.
template <bool MASKED>
__device__ __forceinline__ f32x4 chunk_2x8(const u32x4 cv, uint32_t base, uint32_t mA, uint32_t ok,
                                           const f16x8 (&bx)[8], f32x4 acc) {
    f16x8 a[8], b[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t d = cv[2 * h + (q >> 1)], hw = 2u * (q & 1);
            a[4 * h + q] = as_f16x8(lds16(__builtin_amdgcn_perm(base, d, 0x0c0c0004u | ((hw + mA) << 8))));
            b[4 * h + q] = as_f16x8(lds16(__builtin_amdgcn_perm(base, d, 0x0c0c0005u | ((hw + (mA ^ 1u)) << 8))));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        f16x8 w = a[q], w2 = b[q];
        if constexpr (MASKED) { w = ((ok >> q) & 1u) ? w : f16x8{}; w2 = ((ok >> q) & 1u) ? w2 : f16x8{}; }
        acc = mfma16x16x32(w, bx[q], acc);
        acc = mfma16x16x32(w2, bx[q], acc);
    }
    return acc;
}

// Row-tile geometry of one layer as served by one workgroup.
struct StreamGeo {
    int G, n_slab, n_rt, R, SP, TP;
};

__device__ __forceinline__ StreamGeo stream_geo(int out, int in, int bid, int nwg) {
    StreamGeo g;
    g.G = in / kGroup;
    g.n_slab = (g.G + kSSlab - 1) / kSSlab;
    g.n_rt = (out + 15) / 16;
    g.R = (g.n_rt - bid + nwg - 1) / nwg;
    g.SP = min(kSWaves, g.n_slab);
    g.TP = kSWaves / g.SP;
    return g;
}

// The product for one layer, run by workgroup bid of the nwg that serve it.
// D: steps of codes in flight per wave.
template <int D>
__device__ __forceinline__ void stream_body(const uint8_t* __restrict__ codes, const f16* __restrict__ codebooks,
                                            const f16* __restrict__ scales, f16* __restrict__ y, const int out,
                                            const int bid, const int nwg, const f16* __restrict__ x, const int in,
                                            const int T) {
    extern __shared__ u32x4 smem[];
    const StreamGeo geo = stream_geo(out, in, bid, nwg);
    const int G = geo.G;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lrow = lane & 15, kq = lane >> 4;
    const int sp = wave % geo.SP, tp = wave / geo.SP;
    const int sa = sp * geo.n_slab / geo.SP, sb = (sp + 1) * geo.n_slab / geo.SP;
    const int nW = G / kSSlab;                      // whole slabs of a row
    const int sbw = min(sb, nW);                    // this wave's whole slabs: [sa, sbw)
    const int nsl = max(sbw - sa, 0);
    // this wave's tiles: local j = 0 .. mt - 1 is row tile bid + (tp + TP j) nwg
    const int mt = (wave < geo.SP * geo.TP && tp < geo.R) ? (geo.R - tp + geo.TP - 1) / geo.TP : 0;
    const int total = mt * nsl;                     // steps: tile j = k / nsl, slab sa + k % nsl
    const int XS = ((G + 63) & ~63) + 1;           // 16-byte entries a batch row of x takes in LDS (= 1 mod 16)
    const int xslots = (T * XS + 63) & ~63;
    const int nred = geo.SP + 1;                    // partials per tile: the slab parts, then the ragged slab
    float* red = reinterpret_cast<float*>(smem + kSCbBytes / 16 + xslots);
    const uint16_t* c16 = reinterpret_cast<const uint16_t*>(codes);

    auto tile_row0 = [&](int j) { return (bid + (tp + geo.TP * j) * nwg) * 16; };
    // Codes of slab s of local tile j for this lane: rows past the layer are clamped
    // into it (their outputs are never written), and a chunk of 8 groups past the
    // row (G % 8 == 0) to the row's last chunk (its products are masked).
    auto load_codes = [&](int j, int s) -> u32x4 {
        const int row = min(tile_row0(j) + lrow, out - 1);
        return load16(c16 + (size_t)row * G + min(s * kSSlab + 8 * kq, G - 8));
    };

    // Ring slot d holds the codes of step k0 + d.  Every step uses its slot
    // unconditionally and then refills it with step k + D (a step past the end
    // reloads a valid chunk), so each slot is one register set redefined after
    // its last use, and the compiler's waits are for the oldest load only.
    u32x4 ring[D];
    int jp = 0, spf = sa;   // step whose codes are loaded next
    if (total > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            ring[d] = load_codes(min(jp, mt - 1), spf);
            if (++spf == sbw) { spf = sa; ++jp; }
        }
    }

    // Codebooks: 16-byte slot (2 k + m) 8 + r holds codeword k of codebook m.
#pragma unroll
    for (int it = 0; it < kSCbBytes / 16 / kSThreads; ++it) {
        const int km = (it * kSThreads + tid) / kSRepl;
        __builtin_amdgcn_global_load_lds(
            (const void*)(codebooks + (size_t)((km & 1) * kCodewords2x8 + (km >> 1)) * kGroup),
            lds_ptr(smem + it * kSThreads + wave * kWave), 16, 0, 0);
    }
    // x: entry b XS + j (batch row b, group j) after the codebooks; entries past
    // the end of a row's last 64-entry chunk repeat its last group.  XS = 1 mod 16,
    // so the lanes of the T batch columns that read one group of their rows
    // together hit T distinct 16-byte bank groups.
    {
        const int nch = (G + kWave - 1) / kWave;   // 64-entry chunks a row
        for (int c = wave; c < T * nch; c += kSWaves) {
            const int b = c / nch, j = min((c - b * nch) * kWave + lane, G - 1);
            __builtin_amdgcn_global_load_lds((const void*)(x + (size_t)b * in + (size_t)j * kGroup),
                                             lds_ptr(smem + kSCbBytes / 16 + b * XS + (c - b * nch) * kWave), 16, 0, 0);
        }
    }
    // partials start at zero (a wave with no steps leaves its slots untouched)
    for (int e = tid; e < geo.R * nred * 16 * T; e += kSThreads) red[e] = 0.f;
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    __syncthreads();

    const uint32_t mA = (lane >> 3) & 1u, r16 = (lane & 7u) * 16u;
    const uint32_t base = (r16 + 128u * mA) | ((r16 + 128u * (mA ^ 1u)) << 8);
    const int xrow = min(lrow, T - 1);   // batch columns past the batch repeat the last row (discarded)
    const uint32_t xlane = (uint32_t)kSCbBytes + 16u * (uint32_t)(xrow * XS + 8 * kq);
    // lane (kq, lrow), lrow < T, holds rows 4 kq + r of batch column lrow of a tile
    auto write_partial = [&](int j, int slot, const f32x4& acc) {
        const int i = tp + geo.TP * j;
        if (lrow < T) {
#pragma unroll
            for (int r = 0; r < 4; ++r) red[((i * nred + slot) * 16 + 4 * kq + r) * T + lrow] = acc[r];
        }
    };

    int jc = 0, sc = sa;   // step being consumed
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < total; k0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            // a step past the end (the last round may be short) only refills its slot
            const bool real = k0 + d < total;
            if (real) {
                f16x8 bx[8];   // batch columns past the batch are left unset (their outputs are discarded)
                if (lrow < T) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) bx[q] = as_f16x8(lds16(xlane + 16u * (uint32_t)(sc * kSSlab + q)));
                }
                acc = chunk_2x8<false>(ring[d], base, mA, 0u, bx, acc);
            }
            ring[d] = load_codes(min(jp, mt - 1), spf);
            if (++spf == sbw) { spf = sa; ++jp; }
            if (real && sc == sbw - 1) {   // the tile's last whole slab of this wave
                write_partial(jc, sp, acc);
                acc = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            if (++sc == sbw) { sc = sa; ++jc; }
        }
    }
    // The ragged last slab (G % 32 != 0), masked, by the waves whose range holds it.
    if (sb > nW) {
        for (int j = 0; j < mt; ++j) {
            const u32x4 cv = load_codes(j, nW);
            f16x8 bx[8];
            uint32_t ok = 0u;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int grp = nW * kSSlab + 8 * kq + q;
                ok |= grp < G ? (1u << q) : 0u;
                bx[q] = as_f16x8(lds16(xlane + 16u * (uint32_t)(min(grp, G - 1) - 8 * kq)));
            }
            write_partial(j, geo.SP, chunk_2x8<true>(cv, base, mA, ok, bx, f32x4{0.f, 0.f, 0.f, 0.f}));
        }
    }
    __syncthreads();
    for (int e = tid; e < geo.R * 16 * T; e += kSThreads) {
        const int i = e / (16 * T), rr = (e / T) % 16, col = e % T;
        const int row = (bid + i * nwg) * 16 + rr;
        if (row < out) {
            float sum = 0.f;
            for (int q = 0; q < nred; ++q) sum += red[((i * nred + q) * 16 + rr) * T + col];
            y[(size_t)col * out + row] = (f16)(sum * (float)scales[row]);
        }
    }
}

template <int D>
// One workgroup of 16 waves a CU (its LDS): at most 4 waves a SIMD, so the compiler
// may use up to 128 registers a lane instead of packing for a higher occupancy.
__global__ __launch_bounds__(kSThreads) __attribute__((amdgpu_waves_per_eu(1, 4))) void gemv_stream_kernel(const uint8_t* __restrict__ codes,
                                                                const f16* __restrict__ codebooks,
                                                                const f16* __restrict__ scales, f16* __restrict__ y,
                                                                int out, const f16* __restrict__ x, int in, int T) {
    stream_body<D>(codes, codebooks, scales, y, out, (int)blockIdx.x, (int)gridDim.x, x, in, T);
}

// Several layers that share x; the workgroup's layer is found as in gemv_fused_kernel.
template <int D>
__global__ __launch_bounds__(kSThreads) __attribute__((amdgpu_waves_per_eu(1, 4))) void gemv_stream_fused_kernel(const GemvLayers L, const f16* __restrict__ x,
                                                                      int in, int T) {
    int li = 0, wg0 = 0, wg1 = L.wg_end[0];
#pragma unroll
    for (int i = 0; i + 1 < kGemvMaxLayers; ++i) {
        const bool past = i + 1 < L.n && (int)blockIdx.x >= L.wg_end[i];
        li += past ? 1 : 0;
        wg0 = past ? L.wg_end[i] : wg0;
        wg1 = past ? L.wg_end[i + 1] : wg1;
    }
    stream_body<D>(static_cast<const uint8_t*>(L.codes[li]), static_cast<const f16*>(L.codebooks[li]),
                    static_cast<const f16*>(L.scales[li]), static_cast<f16*>(L.y[li]), L.out[li],
                    (int)blockIdx.x - wg0, wg1 - wg0, x, in, T);
}

template <int D>
hipError_t launch_d(const GemvLayers& layers, const void* x, int in, int T, size_t lds, hipStream_t stream) {
    const bool fused = layers.n > 1;
    const void* kern = fused ? (const void*)gemv_stream_fused_kernel<D> : (const void*)gemv_stream_kernel<D>;
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int grid = layers.wg_end[layers.n - 1];
    if (fused)
        hipLaunchKernelGGL((gemv_stream_fused_kernel<D>), dim3(grid), dim3(kSThreads), lds, stream, layers,
                           (const f16*)x, in, T);
    else
        hipLaunchKernelGGL((gemv_stream_kernel<D>), dim3(grid), dim3(kSThreads), lds, stream,
                           static_cast<const uint8_t*>(layers.codes[0]), static_cast<const f16*>(layers.codebooks[0]),
                           static_cast<const f16*>(layers.scales[0]), static_cast<f16*>(layers.y[0]), layers.out[0],
                           (const f16*)x, in, T);
    return hipGetLastError();
}

}  // namespace

// LDS bytes of the streaming product for layers whose workgroups are dealt
// (wg_end filled), or 0 if it does not serve them: batch above 4, rows of codes
// not 16-byte aligned, more LDS than a workgroup may hold, or a single slab step
// per wave (there its longer prologue, x staged before the first product, costs
// more than the streaming saves: 4096x4096 at batch 1 takes 6.0 us against 5.9
// on gemv_kernel; from two steps on it is the faster kernel, e.g. 1024x8192 6.5
// against 7.0 and 8192x8192 9.5 against 10.3).  At batch 3-4, where x takes
// twice as long to stage, it needs four steps a wave: 11008x4096 (three) takes
// 9.1 us against 9.0, 8192x8192 (four) 10.0 against 10.2, 28672x8192 21.5
// against 28.3.
size_t gemv_stream_lds(const GemvLayers& layers, int64_t in, int64_t batch) {
    if (batch < 1 || batch > kSMaxT || in % 64 != 0 || in <= 0) return 0;
    const int G = (int)(in / kGroup), n_slab = (G + kSSlab - 1) / kSSlab;
    const int SP = std::min(kSWaves, n_slab);
    int rmax = 0, wg0 = 0;
    for (int l = 0; l < layers.n; ++l) {
        const int n_rt = (layers.out[l] + 15) / 16, w = layers.wg_end[l] - wg0;
        wg0 = layers.wg_end[l];
        rmax = std::max(rmax, (n_rt + w - 1) / w);
    }
    if ((int64_t)rmax * n_slab < (batch > 2 ? kSMinSteps34 : kSMinSteps) * kSWaves) return 0;
    const size_t xslots = (size_t)((batch * (((G + 63) & ~63) + 1) + 63) & ~63);
    const size_t lds = (size_t)kSCbBytes + xslots * 16 + (size_t)rmax * (SP + 1) * 16 * batch * sizeof(float);
    return lds <= (size_t)160 * 1024 ? lds : 0;
}

hipError_t launch_gemv_stream(const GemvLayers& layers, const void* x, int64_t in, int64_t batch, size_t lds,
                              hipStream_t stream) {
    return launch_d<kSRing>(layers, x, (int)in, (int)batch, lds, stream);
}

}  // namespace aqlm
