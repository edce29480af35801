// Prefill product on decoded weights:  Y[t][i] = sum_k X[t][k] W16[i][k].
//
// "The AQLM Quantization Algorithm, Explained", Figure 2 of the MCQ section:
// at inference the product with the activations runs on dequantized
// half-precision weights, each the sum of the selected codewords times the
// row scale.  The two-pass prefill path first writes those weights once
// (decode_kernel, bit-exact fp16, the scale already applied) and then runs
// this dense fp16 matrix-core product over them.  Against the fused kernels,
// which decode every W tile again for each 256-token tile, it trades 2 bytes
// per weight of HBM traffic (written once, read once per XCD) for decoding
// each weight once.
//
// A workgroup owns a 256-token x 128-row output tile and walks k in steps of
// 64 inputs, each split into two k-halves of 32 for the products.  Twelve
// waves play two roles:
//   8 consumer waves  each own a 64x64 piece: they read 16-byte fragments from
//                     LDS and run 16x16x32 fp16 matrix-core products with fp32
//                     accumulators, and issue no global load;
//   4 loader waves    copy the X and W tiles of each step straight from global
//                     memory into LDS (direct-to-LDS loads), 12 loads a wave.
// With the copies in the consumer waves instead (6 loads each) the product took
// 10-13 % longer; with two loader waves, 6-9 % longer.
//
// Pipeline (one barrier per step; B_k is the barrier that ends step k):
//   step k : loaders load the X and W tiles of step k+2 (whole rows of 128
//            bytes); consumers read half 0 of step k while multiplying half 1
//            of step k-1, then read half 1 of step k while multiplying half 0;
//            B_k: the loaders' loads issued before step k have landed and the
//            consumers' fragment reads are done.
// X and W keep three whole-step stages each: 96 + 48 = 144 KB of LDS.  The
// products run in the same order as a plain k loop, so the skew changes no
// result.
//
// LDS layout of a stage: row r holds the 8 chunks (16 bytes each) of its 64
// inputs; chunk c sits in slot 8r + (c ^ ((r >> 1) & 7)).  A direct-to-LDS
// load writes 64 consecutive slots, 8 whole rows, so each load reads 8 full
// 128-byte lines (loading the two halves of a row at different times, 16 rows
// of 64 bytes per load, was measured 15-25 % slower).  The 16 lanes of a
// fragment read (16 consecutive rows, one chunk) hit 16 distinct 16-byte bank
// groups.
//
// Epilogue (out % 8 == 0): after a last barrier each consumer wave passes its 64x64 tile
// through LDS and stores whole 128-byte rows of y, 16 bytes per lane.
//
// Tile order: consecutive workgroups go to different XCDs, so workgroup b
// takes tile (b % 8) * per + b / 8 of the token-fastest tile order.  Each XCD
// then holds a contiguous run of row tiles with all their token tiles: its L2
// keeps its own W tiles, and the X tiles that its concurrent workgroups share.
#include "aqlm_device.h"
#include "aqlm_launch.h"

namespace aqlm {

namespace {

constexpr int kDenseBM = 256;                // tokens per tile
constexpr int kDenseBN = 128;                // output rows per tile
constexpr int kDenseWaves = 8;                // consumer waves: the products
constexpr int kDenseLoaders = 4;              // loader waves: the global-to-LDS copies
constexpr int kDenseThreads = 64 * (kDenseWaves + kDenseLoaders);
constexpr int kDenseXStage = kDenseBM * 8;   // 16-byte slots of one X stage (a whole 64-input step)
constexpr int kDenseWStage = kDenseBN * 8;   // 16-byte slots of one W stage
constexpr int kDenseStages = 3;
constexpr int kDenseWOff = kDenseStages * kDenseXStage;
constexpr size_t kDenseLds = (size_t)(kDenseWOff + kDenseStages * kDenseWStage) * 16;
static_assert(kDenseLds <= 163840, "LDS budget");
constexpr int kXcds = 8;                     // tile order only; any count gives correct results

// loads a loader wave issues per step: 8 of X (64 rows), 4 of W (32 rows)
constexpr int kDenseLoadsPerStep = 12;

__device__ __forceinline__ int stage_slot(int r, int c) { return 8 * r + (c ^ ((r >> 1) & 7)); }

// B_{k-1}: every load issued before the previous step has landed (the previous
// step's own stay in flight), every LDS read of the workgroup is done.
__device__ __forceinline__ void step_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kDenseLoadsPerStep));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kDenseThreads) void gemm_dense_kernel(const f16* __restrict__ x,
                                                                   const f16* __restrict__ w, f16* __restrict__ y,
                                                                   int out, int in, int T, int n_tt, int n_tiles,
                                                                   int per_xcd) {
    extern __shared__ u32x4 smem[];
    u32x4* Xs = smem;                 // [stage 3][kDenseXStage]
    u32x4* Ws = smem + kDenseWOff;    // [stage 3][kDenseWStage]
    const int tile = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (tile >= n_tiles) return;      // the whole workgroup: the grid is rounded up to kXcds * per_xcd
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lw = wave - kDenseWaves;   // loader index (loader waves only)
    const int n0 = (tile / n_tt) * kDenseBN;
    const int t0 = (tile % n_tt) * kDenseBM;
    const int n_k = in / 64;          // the launcher guarantees in % 64 == 0

    // The tiles of step j into stage j % 3.  Load q writes slots 64 q .. 64 q + 63:
    // lane l fills slot 64 q + l, which holds chunk (l % 8) ^ ((r >> 1) & 7) of row
    // r = 8 q + l / 8, so the 8 lanes of a row read its whole 128-byte line.
    const int rsub = lane >> 3;
    auto load_step = [&](int j) {
        const int jc = min(j, n_k - 1);
        u32x4* dx = Xs + (j % kDenseStages) * kDenseXStage;
        u32x4* dw = Ws + (j % kDenseStages) * kDenseWStage;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = 8 * lw + i;
            const int r = 8 * q + rsub;
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            const int tok = min(t0 + r, T - 1);
            __builtin_amdgcn_global_load_lds((const void*)(x + (size_t)tok * in + (size_t)(8 * jc + c) * kGroup),
                                             lds_ptr(dx + 64 * q), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = 4 * lw + i;
            const int r = 8 * q + rsub;
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            const int row = min(n0 + r, out - 1);
            __builtin_amdgcn_global_load_lds((const void*)(w + (size_t)row * in + (size_t)(8 * jc + c) * kGroup),
                                             lds_ptr(dw + 64 * q), 16, 0, 0);
        }
    };

    const int wm = wave >> 1, wn = wave & 1;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // fragments of half h of step j: lane l holds A[l%16][8(l/16)..] and B[8(l/16)..][l%16]
    auto read_frags = [&](int j, int h, f16x8 (&a)[4], f16x8 (&b)[4]) {
        const u32x4* xb = Xs + (j % kDenseStages) * kDenseXStage;
        const u32x4* wb = Ws + (j % kDenseStages) * kDenseWStage;
        const int cc = 4 * h + (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = as_f16x8(xb[stage_slot(wm * 64 + i * 16 + (lane & 15), cc)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = as_f16x8(wb[stage_slot(wn * 64 + i * 16 + (lane & 15), cc)]);
    };
    // 16 products of one k-half, one fragment read slotted between every two of them
    // (product, read, product: 1-7 % faster than read, product, product)
    auto mma16 = [&](const f16x8 (&a)[4], const f16x8 (&b)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix product
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix product
        }
    };
    if (lw >= 0) {
        // loader: the same barriers as the consumers, the loads of step k+2 after B_{k-1}
        // (stage (k-1) % 3: step k-1 was read before B_{k-1})
        load_step(0);
        load_step(1);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));   // steps 0 and 1 landed
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        load_step(2);
        for (int k = 1; k < n_k; ++k) {
            step_barrier();
            load_step(k + 2);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));   // no load in flight into the epilogue's LDS
        if (out % 8 == 0) {
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        return;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    f16x8 a0[4], b0[4], a1[4], b1[4];
    // step 0: both halves of stage 0 read, half 0 multiplied
    __builtin_amdgcn_sched_barrier(0);
    read_frags(0, 0, a0, b0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    read_frags(0, 1, a1, b1);
    mma16(a0, b0);
    for (int k = 1; k < n_k; ++k) {
        step_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(k, 0, a0, b0);
        mma16(a1, b1);          // half 1 of step k-1
        __builtin_amdgcn_sched_barrier(0);
        read_frags(k, 1, a1, b1);
        mma16(a0, b0);          // half 0 of step k
    }
    mma16(a1, b1);              // half 1 of the last step

    if (out % 8 == 0) {
        // Every load of every wave has landed and every fragment read is done, so the
        // stages are free: each wave's 64x64 tile goes through LDS (fp16, rows of 64 + 8
        // padding) and leaves as 16-byte stores, 8 lanes per 128-byte row of y.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        constexpr int kEpiStride = 72;
        f16* etile = reinterpret_cast<f16*>(smem) + wave * 64 * kEpiStride;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    etile[(i * 16 + 4 * (lane >> 4) + r) * kEpiStride + j * 16 + (lane & 15)] = (f16)acc[i][j][r];
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        const int c8 = (lane & 7) * 8;
        const int col = n0 + wn * 64 + c8;
        if (col < out) {   // out % 8 == 0: a chunk is wholly inside or wholly outside
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int rr = it * 8 + (lane >> 3);
                const int tok = t0 + wm * 64 + rr;
                if (tok < T)
                    *reinterpret_cast<u32x4*>(y + (size_t)tok * out + col) =
                        *reinterpret_cast<const u32x4*>(etile + rr * kEpiStride + c8);
            }
        }
        return;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));   // no LDS load in flight at exit

    // rows not a multiple of 8: lane holds D[4*(l/16)+r][l%16] of block (i, j), stored directly
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (col >= out) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = t0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
                if (tok < T) y[(size_t)tok * out + col] = (f16)acc[i][j][r];
            }
    }
}

}  // namespace

hipError_t launch_gemm_dense(const void* x, const void* w16, void* y, int64_t out, int64_t in, int64_t batch,
                             hipStream_t stream) {
    if (in % 64 != 0) return hipErrorInvalidValue;
    if (out == 0 || batch == 0) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute((const void*)gemm_dense_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDenseLds);
    if (e != hipSuccess) return e;
    const int64_t n_tt = (batch + kDenseBM - 1) / kDenseBM;
    const int64_t n_tiles = ((out + kDenseBN - 1) / kDenseBN) * n_tt;
    const int64_t per = (n_tiles + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(gemm_dense_kernel, dim3((unsigned)(per * kXcds)), dim3(kDenseThreads), kDenseLds, stream,
                       (const f16*)x, (const f16*)w16, (f16*)y, (int)out, (int)in, (int)batch, (int)n_tt,
                       (int)n_tiles, (int)per);
    return hipGetLastError();
}

}  // namespace aqlm
