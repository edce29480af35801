// Prefill product for the 2x8 scheme with a role-split software pipeline:
//   Y[t][i] = s[i] * sum_k X[t][k] Wc[i][k],  Wc[i][8j+u] = C0[b0][u] + C1[b1][u].
// The same kernel serves the other 2-bit schemes whose codes also take 2 bytes
// per 8 inputs at the same places ("Key AQLM quantization parameters"): 1x8 g4,
// where the 8 weights of a piece are two 4-entry codewords, Wc[i][8j+u] =
// C0[b_{2j}][u] for u < 4 and C0[b_{2j+1}][u-4] above, and 4x8 g16, where a
// group of 16 inputs is the sum of four 16-entry codewords (4 code bytes).  It
// also serves 1x16, whose 16-bit codes take the same 2 bytes per 8 inputs and
// whose single codeword is the weight piece: its 1 MiB codebook does not fit
// LDS and is gathered from L2 (see the producers below).
//
// "The AQLM Quantization Algorithm, Explained", Figure 2 of the MCQ section:
// the product runs on dequantized half-precision weights, each built from one
// codeword per codebook.  This kernel is the fast path for in % 64 == 0; the
// general kernel in gemm.hip handles every other shape.
//
// A workgroup owns a 256-token x 128-row output tile and walks k in steps of
// 64 inputs (8 groups).  Each step is split into two k-halves of 32 inputs.
// Twelve waves play two roles:
//
//   8 consumer waves  each own a 64x64 piece of the tile.  They copy X
//                     straight from global memory into LDS (direct-to-LDS
//                     loads), read 16-byte fragments and run 16x16x32 fp16
//                     matrix-core products with fp32 accumulators.
//   4 producer waves  stream the codes of the tile far ahead into an LDS ring
//                     (also direct-to-LDS) and decode W from the LDS copy of
//                     the two codebooks into LDS as fp16.
//
// Only code loads go through the producers' vector-memory counter, so they can
// run kRing steps ahead; the consumers' counter only holds X loads.  Both
// counters retire in issue order, which is why the two kinds of loads live in
// different waves.  For 1x16 the producers split once more: two waves stream the
// codes (kept three steps ahead of the gathers) and two gather the codewords (8 a
// lane a step) one step before they write them to W, so that waiting for a gather
// never waits for code loads issued after it.  At 2048 tokens this is 15-17 %
// faster than the general kernel; gathering in the step that writes, 7-9 %;
// gathering two steps ahead, 13-15 %; the code loads moved to the consumers with
// four gathering waves, 2-4 %.
//
// Pipeline (one barrier per step; B_k is the barrier that ends step k):
//   consumer step k : load the X tile of step k+2 (whole 128-byte rows);
//                     read half 0 of step k, multiply half 1 of step k-1;
//                     read half 1 of step k, multiply half 0 of step k;
//                     B_k waits for every X load issued before step k.
//   producer step k : load the codes of step k+kRing;
//                     decode the whole W tile of step k+1;
//                     B_k waits for the codes of step k+2.
// X tiles thus have two steps to arrive, code loads about kRing-2.  X keeps
// three stages, W two (a W tile is written one step before it is read), the
// code ring kRing steps: 96 + 32 + 24 + 8 (codebooks; 2 KB for 1x8 g4) = 160 KB.  4x8 g16
// keeps two X stages next to its 32 KB of codebooks (64 + 32 + 24 + 32 = 152 KB), so its X
// tiles have one step to arrive.  The products run in the order of a plain k loop.
//
// Epilogue (out % 8 == 0): producers and consumers meet at a last barrier; then
// each consumer wave passes its scaled 64x64 tile through LDS and stores whole
// 128-byte rows of y, 16 bytes per lane (2-byte stores per lane wrote 1.47x the
// bytes of y on 11008 rows: partial lines).
//
// LDS layout of a stage: row r holds the 8 chunks (16 bytes each) of its 64
// inputs; chunk c sits in slot 8r + (c ^ ((r >> 1) & 7)).  A direct-to-LDS
// load writes 64 consecutive slots, 8 whole rows, so each X load reads 8 full
// 128-byte lines (loading the two halves of a row at different times, 16 rows
// of 64 bytes per load, was measured 16-21 % slower).  The 16 lanes of a
// fragment read (16 consecutive rows, one chunk) hit 16 distinct bank groups.
#include "aqlm_device.h"
#include "aqlm_launch.h"

namespace aqlm {

namespace {

constexpr int kPipeBM = 256;                 // tokens per tile
constexpr int kPipeBN = 128;                 // output rows per tile
constexpr int kPipeConsumers = 8;            // consumer waves
constexpr int kPipeProducers = 4;            // producer waves
constexpr int kPipeThreads = 64 * (kPipeConsumers + kPipeProducers);
constexpr int kPipeXStage = kPipeBM * 8;     // 16-byte slots of one X stage (a whole step)
constexpr int kPipeWStage = kPipeBN * 8;     // 16-byte slots of one W stage
constexpr int kPipeWStages = 2;
constexpr int kPipeRing = 12;                // steps of codes held in LDS
// codebook slots: 2x8 codeword k of codebook m at 256 m + k (the codebooks one after the
// other: a producer read of one codebook then spreads its lanes over all 16 bank groups,
// where interleaved codebooks left it 8; 4096^2 at 2048 tokens 80.4 -> 74.9 us); 1x8 g4
// codeword k in 8-byte slot k; 4x8 g16 half h (8 entries) of codeword k of codebook m at
// 1024 h + 256 m + k (32 KB).
template <int SCHEME>
constexpr int pipe_cb_slots() {
    return SCHEME == kScheme2x8 ? 2 * kCodewords2x8 : SCHEME == kSchemeB8M4 ? 8 * kCodewords2x8
         : SCHEME == kScheme1x16 ? 0 : kCodewords2x8 / 2;
}
// X stages: three (X loads get two steps to land), or two for 4x8 g16, whose 32 KB of
// codebooks leave no room for a third (its X loads get one step).
template <int SCHEME>
constexpr int pipe_x_stages() { return SCHEME == kSchemeB8M4 ? 2 : 3; }
template <int SCHEME>
struct PipeLayout {   // offsets in 16-byte slots
    static constexpr int kX = 0;
    static constexpr int kW = kX + pipe_x_stages<SCHEME>() * kPipeXStage;
    static constexpr int kRing = kW + kPipeWStages * kPipeWStage;
    static constexpr int kCb = kRing + kPipeRing * kPipeBN;
    static constexpr size_t kBytes = (size_t)(kCb + pipe_cb_slots<SCHEME>()) * 16;
    static_assert(kBytes <= 163840, "LDS budget");
};

__device__ __forceinline__ int stage_slot(int r, int c) { return 8 * r + (c ^ ((r >> 1) & 7)); }

template <int SCHEME>
__global__ __launch_bounds__(kPipeThreads) void gemm_pipe_2x8_kernel(
    const uint8_t* __restrict__ codes, const f16* __restrict__ codebooks,
    const f16* __restrict__ scales, const f16* __restrict__ x, f16* __restrict__ y,
    int out, int in, int T) {
    extern __shared__ u32x4 smem[];
    using Lay = PipeLayout<SCHEME>;
    constexpr int kXS = pipe_x_stages<SCHEME>();
    u32x4* Xs = smem + Lay::kX;         // [stage kXS][kPipeXStage]
    u32x4* Ws = smem + Lay::kW;         // [stage 2][kPipeWStage]
    u32x4* ring = smem + Lay::kRing;    // [kPipeRing][row 128] : the codes of a row's 64 inputs, 16 bytes
    u32x4* cb = smem + Lay::kCb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = in / kGroup;
    const int n_k = G / 8;                          // the launcher guarantees in % 64 == 0
    const int n_tt = (T + kPipeBM - 1) / kPipeBM;
    const int n0 = (int)(blockIdx.x / n_tt) * kPipeBN;
    const int t0 = (int)(blockIdx.x % n_tt) * kPipeBM;

    if constexpr (SCHEME == kScheme2x8) {
        for (int j = tid; j < pipe_cb_slots<SCHEME>(); j += kPipeThreads)
            cb[j] = load16(codebooks + (size_t)j * kGroup);
    } else if constexpr (SCHEME == kSchemeB8M4) {
        // slot j = 1024 h + km (km = 256 m + k): entries 8 h .. 8 h + 7 of codeword km
        for (int j = tid; j < pipe_cb_slots<SCHEME>(); j += kPipeThreads)
            cb[j] = load16(codebooks + (size_t)(j & 1023) * 16 + (j >> 10) * 8);
    } else if constexpr (SCHEME == kSchemeB8M1) {
        u32x2* cb8 = reinterpret_cast<u32x2*>(cb);
        for (int j = tid; j < kCodewords2x8; j += kPipeThreads)
            cb8[j] = *reinterpret_cast<const u32x2*>(codebooks + (size_t)j * 4);
    }

    if (wave >= kPipeConsumers) {
        // ------------------------------ producers ------------------------------
        const int pw = wave - kPipeConsumers;
        const uint32_t* c32 = reinterpret_cast<const uint32_t*>(codes);
        // the 2 KB of codes of step j: dword d of the slot is dword d & 3 of row d >> 2
        auto load_codes = [&](int j) {
            const int jc = min(j, n_k - 1);
            uint32_t* slot = reinterpret_cast<uint32_t*>(ring + (j % kPipeRing) * kPipeBN);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int d = (2 * pw + i) * 64 + lane;
                const int row = min(n0 + (d >> 2), out - 1);
                __builtin_amdgcn_global_load_lds((const void*)(c32 + (size_t)row * (G / 2) + jc * 4 + (d & 3)),
                                                 lds_ptr(slot + (2 * pw + i) * 64), 4, 0, 0);
            }
        };
        // thread p decodes chunks c0 .. c0+3 of row r of step j; every LDS read is
        // issued before the first write so the lookups overlap
        const int p = tid - 64 * kPipeConsumers;
        const int r = p >> 1, c0 = 4 * (p & 1);
        auto decode_step = [&](int j) {
            const uint32_t* cr = reinterpret_cast<const uint32_t*>(ring + (j % kPipeRing) * kPipeBN + r);
            const uint32_t ca = cr[c0 >> 1], cw = cr[(c0 >> 1) + 1];
            u32x4* d = Ws + (j % kPipeWStages) * kPipeWStage;
            if constexpr (SCHEME == kScheme2x8) {
                f16x8 e[8];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    e[2 * q] = as_f16x8(cb[(ca >> (16 * q)) & 0xff]);
                    e[2 * q + 1] = as_f16x8(cb[kCodewords2x8 + ((ca >> (16 * q + 8)) & 0xff)]);
                    e[4 + 2 * q] = as_f16x8(cb[(cw >> (16 * q)) & 0xff]);
                    e[5 + 2 * q] = as_f16x8(cb[kCodewords2x8 + ((cw >> (16 * q + 8)) & 0xff)]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) d[stage_slot(r, c0 + q)] = as_u32x4(e[2 * q] + e[2 * q + 1]);
            } else if constexpr (SCHEME == kSchemeB8M4) {
                // piece c0 + q (c0 even): half q % 2 of group c0 / 2 + q / 2 (16 inputs), whose
                // 4 code bytes are dword c0 / 2 + q / 2 of the row's step; the four codewords'
                // halves added in fp16 from codebook 0 up
                f16x8 t[4][4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t cd = q < 2 ? ca : cw;
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        t[q][m] = as_f16x8(cb[1024 * (q & 1) + 256 * m + ((cd >> (8 * m)) & 0xff)]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    d[stage_slot(r, c0 + q)] = as_u32x4(((t[q][0] + t[q][1]) + t[q][2]) + t[q][3]);
            } else {
                // piece c0 + q: groups 2 (c0 + q) and 2 (c0 + q) + 1, one byte each
                const u32x2* cb8 = reinterpret_cast<const u32x2*>(cb);
                u32x2 e[8];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    e[2 * q] = cb8[(ca >> (16 * q)) & 0xff];
                    e[2 * q + 1] = cb8[(ca >> (16 * q + 8)) & 0xff];
                    e[4 + 2 * q] = cb8[(cw >> (16 * q)) & 0xff];
                    e[5 + 2 * q] = cb8[(cw >> (16 * q + 8)) & 0xff];
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    d[stage_slot(r, c0 + q)] = u32x4{e[2 * q][0], e[2 * q][1], e[2 * q + 1][0], e[2 * q + 1][1]};
            }
        };
        if constexpr (SCHEME == kScheme1x16) {
            // The 65536-entry codebook stays in L2.  Two of the producer waves stream the codes
            // into the ring (4 loads of 256 bytes each a step); the other two gather each row's 8
            // codewords of a step from L2, one step before writing them to the W tile.  Each
            // wave's vector-memory counter then holds one kind of load, so the gathers are
            // waited for without waiting for the code loads issued after them.
            if (pw < 2) {
                auto load_ring = [&](int j) {
                    const int jc = min(j, n_k - 1);
                    uint32_t* slot = reinterpret_cast<uint32_t*>(ring + (j % kPipeRing) * kPipeBN);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int d = (4 * pw + i) * 64 + lane;
                        const int row = min(n0 + (d >> 2), out - 1);
                        __builtin_amdgcn_global_load_lds((const void*)(c32 + (size_t)row * (G / 2) + jc * 4 + (d & 3)),
                                                         lds_ptr(slot + (4 * pw + i) * 64), 4, 0, 0);
                    }
                };
#pragma unroll
                for (int j = 0; j < kPipeRing; ++j) load_ring(j);
                // P1: codes of steps 0 and 1 landed
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(4 * (kPipeRing - 2)) : "memory");
                // P2: codes of step 2 landed
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(4 * (kPipeRing - 3)) : "memory");
                for (int k = 0; k + 1 < n_k; ++k) {
                    load_ring(k + kPipeRing);   // replaces step k's codes, gathered before B_{k-2}
                    // B_k: codes of step k+3 landed
                    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(4 * (kPipeRing - 3)) : "memory");
                }
            } else {
                const int gr = (pw - 2) * 64 + lane;   // the W row this lane writes
                // the codewords of a step are gathered one step before they are written
                const f16* cbl = codebooks;
                asm volatile("" : "+s"(cbl));   // loads through a laundered pointer stay where they are written
                auto gather = [&](int j, u32x4 (&e)[8]) {
                    const u32x4 cv = ring[(min(j, n_k - 1) % kPipeRing) * kPipeBN + gr];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const uint32_t code = (cv[q >> 1] >> (16 * (q & 1))) & 0xffffu;
                        e[q] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(
                            (uintptr_t)(cbl + (size_t)code * kGroup));
                    }
                };
                auto write = [&](int j, const u32x4 (&e)[8]) {
                    u32x4* d = Ws + (j % kPipeWStages) * kPipeWStage;
#pragma unroll
                    for (int q = 0; q < 8; ++q) d[stage_slot(gr, q)] = e[q];
                };
                u32x4 ea[8], eb[8];
                // P1: codes of steps 0 and 1 landed (the ring waves' side)
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                gather(0, ea);
                gather(1, eb);
                write(0, ea);
                // P2: W(0) written; codes of step 2 landed
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                // step k: gather step k+2 (its codes landed at B_{k-1}), write step k+1
                auto round = [&](int k, u32x4 (&next)[8], u32x4 (&cur)[8]) {
                    gather(k + 2, next);
                    write(k + 1, cur);   // stage (k+1) % 2: step k-1's W was read before B_{k-1}
                    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                };
                int k = 0;
                for (; k + 2 < n_k; k += 2) {   // both register sets every round
                    round(k, ea, eb);
                    round(k + 1, eb, ea);
                }
                if (k + 1 < n_k) round(k, ea, eb);
            }
            if (out % 8 == 0) {
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < kPipeRing; ++j) load_codes(j);
        // P1: codebook copy staged, codes of step 0 landed
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * (kPipeRing - 1)) : "memory");
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        decode_step(0);
        // P2: W(0) written, codes of step 1 landed
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * (kPipeRing - 2)) : "memory");
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        for (int k = 0; k + 1 < n_k; ++k) {
            load_codes(k + kPipeRing);          // replaces step k's codes, decoded before B_{k-1}
            __builtin_amdgcn_sched_barrier(0);
            decode_step(k + 1);                 // stage (k+1) % 2: step k-1's W was read before B_{k-1}
            __builtin_amdgcn_sched_barrier(0);
            // B_k: W(k+1) written, codes of step k+2 landed (issued kPipeRing-2 steps ago or earlier)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * (kPipeRing - 2)) : "memory");
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        }
        if (out % 8 == 0) {   // the consumers' epilogue barrier: LDS is free after it
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no LDS load in flight at exit
        }
        return;
    }

    // ------------------------------ consumers ------------------------------
    const int wm = wave >> 1, wn = wave & 1;
    // X of step j into stage j % kXS: load q writes slots 64q .. 64q+63, lane l the chunk
    // (l % 8) ^ ((rr >> 1) & 7) of row rr = 8q + l/8 (8 whole 128-byte lines per load)
    auto load_x = [&](int j) {
        const int jc = min(j, n_k - 1);
        u32x4* dst = Xs + (j % kXS) * kPipeXStage;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = 4 * wave + i;
            const int rr = 8 * q + (lane >> 3);
            const int c = (lane & 7) ^ ((rr >> 1) & 7);
            const int tok = min(t0 + rr, T - 1);
            __builtin_amdgcn_global_load_lds((const void*)(x + (size_t)tok * in + (size_t)(8 * jc + c) * kGroup),
                                             lds_ptr(dst + 64 * q), 16, 0, 0);
        }
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto read_frags = [&](int j, int h, f16x8 (&a)[4], f16x8 (&b)[4]) {
        const u32x4* xb = Xs + (j % kXS) * kPipeXStage;
        const u32x4* wb = Ws + (j % kPipeWStages) * kPipeWStage;
        const int c = 4 * h + (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = as_f16x8(xb[stage_slot(wm * 64 + i * 16 + (lane & 15), c)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = as_f16x8(wb[stage_slot(wn * 64 + i * 16 + (lane & 15), c)]);
    };
    auto mma16 = [&](const f16x8 (&a)[4], const f16x8 (&b)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {   // product, read, product: 3-7 % faster than read, product, product
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix product
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix product
        }
    };
    load_x(0);
    if constexpr (kXS == 3) load_x(1);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // P1: codebook copy staged
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");     // P2: X(0) (and X(1)) landed, W(0) written
    f16x8 a0[4], b0[4], a1[4], b1[4];
    load_x(kXS - 1);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(0, 0, a0, b0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    read_frags(0, 1, a1, b1);
    mma16(a0, b0);
    for (int k = 1; k < n_k; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        // B_{k-1}: X(k) has landed.  Three stages: the four X loads issued after it, those of
        // step k+1, stay in flight; two stages: X(k) is the last load issued.
        if constexpr (kXS == 3)
            asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        load_x(k + kXS - 1);    // stage (k-1) % kXS: step k-1 was read before B_{k-1}
        __builtin_amdgcn_sched_barrier(0);
        read_frags(k, 0, a0, b0);
        mma16(a1, b1);          // half 1 of step k-1
        __builtin_amdgcn_sched_barrier(0);
        read_frags(k, 1, a1, b1);
        mma16(a0, b0);          // half 0 of step k
    }
    mma16(a1, b1);              // half 1 of the last step
    if (out % 8 == 0) {
        // all loads landed, all fragment reads and W writes done (producers join this
        // barrier): each wave's scaled 64x64 tile goes through LDS and leaves as 16-byte
        // stores, 8 lanes per 128-byte row of y
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        constexpr int kEpiStride = 72;
        f16* etile = reinterpret_cast<f16*>(smem) + wave * 64 * kEpiStride;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int colj = min(n0 + wn * 64 + j * 16 + (lane & 15), out - 1);
            const float s = (float)scales[colj];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    etile[(i * 16 + 4 * (lane >> 4) + rr) * kEpiStride + j * 16 + (lane & 15)] = (f16)(acc[i][j][rr] * s);
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        const int c8 = (lane & 7) * 8;
        const int col = n0 + wn * 64 + c8;
        if (col < out) {
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int r8 = it * 8 + (lane >> 3);
                const int tok = t0 + wm * 64 + r8;
                if (tok < T)
                    *reinterpret_cast<u32x4*>(y + (size_t)tok * out + col) =
                        *reinterpret_cast<const u32x4*>(etile + r8 * kEpiStride + c8);
            }
        }
        return;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no LDS load in flight at exit

    // rows not a multiple of 8: lane holds D[4*(l/16)+r][l%16] of block (i, j), stored directly
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (col >= out) continue;
        const float s = (float)scales[col];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int tok = t0 + wm * 64 + i * 16 + 4 * (lane >> 4) + rr;
                if (tok < T) y[(size_t)tok * out + col] = (f16)(acc[i][j][rr] * s);
            }
    }
}

}  // namespace

template <int SCHEME>
static hipError_t launch_pipe(const void* codes, const void* codebooks, const void* scales, const void* x, void* y,
                              int64_t out, int64_t in, int64_t batch, hipStream_t stream) {
    if (in % 64 != 0) return hipErrorInvalidValue;
    const size_t lds = PipeLayout<SCHEME>::kBytes;
    const hipError_t e = hipFuncSetAttribute((const void*)gemm_pipe_2x8_kernel<SCHEME>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(((out + kPipeBN - 1) / kPipeBN) * ((batch + kPipeBM - 1) / kPipeBM)));
    hipLaunchKernelGGL(gemm_pipe_2x8_kernel<SCHEME>, grid, dim3(kPipeThreads), lds, stream,
                       (const uint8_t*)codes, (const f16*)codebooks, (const f16*)scales, (const f16*)x,
                       (f16*)y, (int)out, (int)in, (int)batch);
    return hipGetLastError();
}

hipError_t launch_gemm_pipe_2x8(const void* codes, const void* codebooks, const void* scales,
                                const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                                hipStream_t stream) {
    return launch_pipe<kScheme2x8>(codes, codebooks, scales, x, y, out, in, batch, stream);
}

hipError_t launch_gemm_pipe_1x8g4(const void* codes, const void* codebooks, const void* scales,
                                  const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                                  hipStream_t stream) {
    return launch_pipe<kSchemeB8M1>(codes, codebooks, scales, x, y, out, in, batch, stream);
}

hipError_t launch_gemm_pipe_1x16(const void* codes, const void* codebooks, const void* scales,
                                 const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                                 hipStream_t stream) {
    return launch_pipe<kScheme1x16>(codes, codebooks, scales, x, y, out, in, batch, stream);
}

hipError_t launch_gemm_pipe_4x8g16(const void* codes, const void* codebooks, const void* scales,
                                   const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                                   hipStream_t stream) {
    return launch_pipe<kSchemeB8M4>(codes, codebooks, scales, x, y, out, in, batch, stream);
}

}  // namespace aqlm
