// Decode-phase product for the 1x16 scheme at batch 1 over "slice lists": the
// codes of a layer regrouped once, at load time, by codebook slice.
//
// "The AQLM Quantization Algorithm, Explained", section "Why and what do we
// quantize?": decoding is memory-bound, and dequantization overhead can eat
// the gain.  For 1x16 (section "Key AQLM quantization parameters": 2^16
// codewords, the slower scheme) that overhead is the lookup: a 16-byte
// codeword gathered from the 1 MiB codebook costs one L2 request, and L2
// requests, not HBM, bound a kernel that gathers per code.
//
// Here the codebook is cut into 8 slices of 8192 codewords (128 KB each), and
// a workgroup holds one slice in LDS, so no lookup leaves the CU.  For that to
// pay, a workgroup must read only the codes of its slice, which the row-major
// code array does not allow; hence the layout built by aqlm_lists_plan and
// aqlm_lists_fill from the plain codes:
//
//   rows form tiles of 64 (lane l of a wave serves row 64 rt + l); the groups
//   j of a row form J blocks of at most 1024 groups (block k starts at
//   k * Gb); for every (slice s, block k, row tile rt) unit, each row lists
//   its codes c with c >> 13 == s and j in block k, in ascending j, as 32-bit
//   entries ((j - k Gb) << 13) | (c & 8191).  The 64 lists of a unit are
//   padded to the longest one, L, with the entry Z << 13 (Z: the block size
//   rounded up to 64; x chunk Z is zero in LDS), and stored step-major:
//   entry t of row l at entries[(off + t) * 64 + l].
//
//   table (uint32): for unit u = (s * J + k) * n_rt + rt, table[2u] = off
//   (in steps of 64 entries) and table[2u + 1] = L; then the total number of
//   steps as a uint64 at word 2 * n_units.
//
// Nothing is lost: the multiset of (row, j, code) triples is the code array.
// The product then reads every entry once (coalesced 256-byte steps), looks
// up its codeword and its 8 activations in LDS, and accumulates in fp32 per
// lane (one row per lane: no cross-lane reduction).  When a row tile's steps
// are split over P waves of a workgroup, their sums are added in LDS in part
// order; every unit then writes one fp32 partial per row, and a second kernel
// adds a row's 8 J partials in a fixed order, applies the scale and rounds to
// fp16 once.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "aqlm_device.h"
#include "aqlm_launch.h"

namespace aqlm {

// Scratch of the allocation-free product (aqlm_linear_gemv_lists_noalloc): the fp32
// partial sums of one layer, kListsScratchBytes at most.  Every GPU holds its own copy
// for the life of the process.  In host code `scratch` only names the symbol; its
// device address comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) float scratch[kListsScratchBytes / 4];

namespace {

constexpr int kSlices = 8;
constexpr int kSliceBits = 13;
constexpr int kSliceWords = 1 << kSliceBits;     // codewords per slice: 128 KB of LDS
constexpr int kListThreads = 1024;
constexpr int kListWaves = kListThreads / kWave;
constexpr int kListRing = 8;                     // entry loads per lane and chunk of steps
constexpr int kListRingBusy = 4;                 // the same on one-ring launches whose every wave has a unit
constexpr int kListLongPart = 64;
// The prologue waits are written as the builtin, not as inline assembly, so that
// the compiler's own wait placement knows what has landed (otherwise it assumes
// the direct-to-LDS fill may still be in flight and waits for every load at the
// top of each product loop).
static_assert(kListRing < 16 && kListRingBusy < 16, "vmcnt field");                // launches whose parts have this many steps use two rings
constexpr int kWgPerSlice = 32;                  // workgroups per (slice, block): 256 in all
constexpr int kReduceParts = 4;                  // threads per row in the partial sum

// 8 fp16 weights times 8 fp16 activations, accumulated in fp32 two products
// at a time (v_dot2_f32_f16, no rounding between the two products).
__device__ __forceinline__ float dot8(const u32x4 w, const u32x4 xv, float acc) {
    const f16x8 a = as_f16x8(w), b = as_f16x8(xv);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f16x2 pa, pb;
        pa[0] = a[2 * q];
        pa[1] = a[2 * q + 1];
        pb[0] = b[2 * q];
        pb[1] = b[2 * q + 1];
        acc = __builtin_amdgcn_fdot2(pa, pb, acc, false);
    }
    return acc;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}

// ---- plan: L of every unit (one wave per unit; lane = row)
__global__ __launch_bounds__(256) void lists_count_kernel(const uint16_t* __restrict__ codes, int out,
                                                          ListsGeo geo, uint32_t* __restrict__ table) {
    const int lane = threadIdx.x & 63;
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= geo.n_units()) return;
    const int rt = (int)(u % geo.n_rt);
    const int k = (int)((u / geo.n_rt) % geo.J);
    const int s = (int)(u / ((int64_t)geo.n_rt * geo.J));
    const int row = rt * 64 + lane;
    const int j0 = k * geo.Gb, j1 = min(geo.G, j0 + geo.Gb);
    int n = 0;
    if (row < out) {
        const uint16_t* c = codes + (size_t)row * geo.G;
        for (int j = j0; j < j1; ++j) n += (c[j] >> kSliceBits) == s;
    }
    n = wave_max(n);
    if (lane == 0) table[2 * u + 1] = (uint32_t)n;
}

// ---- plan: offsets (exclusive prefix of L in unit order) and the total, one workgroup
__global__ __launch_bounds__(1024) void lists_scan_kernel(ListsGeo geo, uint32_t* __restrict__ table) {
    __shared__ uint64_t wsum[16];
    __shared__ uint64_t carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = geo.n_units();
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int64_t base = 0; base < n; base += 1024) {
        const int64_t u = base + tid;
        const uint64_t L = u < n ? table[2 * u + 1] : 0;
        uint64_t incl = L;   // inclusive scan within the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint64_t v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        uint64_t before = carry_s;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        if (u < n) table[2 * u] = (uint32_t)(before + incl - L);
        __syncthreads();
        if (tid == 1023) carry_s = before + incl;
        __syncthreads();
    }
    if (tid == 0) *reinterpret_cast<uint64_t*>(table + 2 * n) = carry_s;
}

// ---- fill: one wave per unit writes its 64 lists, padded to L
__global__ __launch_bounds__(256) void lists_fill_kernel(const uint16_t* __restrict__ codes, int out, ListsGeo geo,
                                                         const uint32_t* __restrict__ table,
                                                         uint32_t* __restrict__ entries, uint64_t cap_steps) {
    const int lane = threadIdx.x & 63;
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= geo.n_units()) return;
    const uint64_t off = table[2 * u], L = table[2 * u + 1];
    if (off + L > cap_steps) return;   // not the table of this layer: leave the entries alone
    const int rt = (int)(u % geo.n_rt);
    const int k = (int)((u / geo.n_rt) % geo.J);
    const int s = (int)(u / ((int64_t)geo.n_rt * geo.J));
    const int row = rt * 64 + lane;
    const int j0 = k * geo.Gb, j1 = min(geo.G, j0 + geo.Gb);
    uint32_t* e = entries + off * 64 + lane;
    uint64_t t = 0;
    if (row < out) {
        const uint16_t* c = codes + (size_t)row * geo.G;
        for (int j = j0; j < j1 && t < L; ++j) {
            const uint32_t code = c[j];
            if ((int)(code >> kSliceBits) == s) {
                e[t * 64] = ((uint32_t)(j - j0) << kSliceBits) | (code & (kSliceWords - 1));
                ++t;
            }
        }
    }
    for (; t < L; ++t) e[t * 64] = (uint32_t)geo.Z << kSliceBits;
}

// Layer of block b from a table of cumulative ends, and the layer's first block
// (branch-free over values already in scalar registers: one round trip to the
// kernel arguments before the layer's own fields).
__device__ __forceinline__ int layer_of(const int* end, int n, int b, int* base) {
    int l = 0, first = 0;
#pragma unroll
    for (int i = 0; i < kGemvMaxLayers - 1; ++i) {
        const bool past = (i < n - 1) & (b >= end[i]);
        l += past;
        first = past ? end[i] : first;
    }
    *base = first;
    return l;
}

// ---- the product: workgroup bid of one layer.  LONG: the parts have many steps (two
// rings of entries in flight); otherwise one ring and a barrier that waits for the fill only.
template <bool LONG, int RING>
__device__ __forceinline__ void lists_product(const uint32_t* __restrict__ table, const uint32_t* __restrict__ entries,
                                              uint64_t cap_steps, const f16* __restrict__ codebook,
                                              const f16* __restrict__ x, float* __restrict__ partial,
                                              const ListsGeo geo, int bid) {
    extern __shared__ u32x4 smem[];
    u32x4* cbs = smem;                 // the slice: kSliceWords codewords
    u32x4* xs = smem + kSliceWords;    // the x block: Z + 1 chunks of 8 fp16, chunk Z = 0
    float* red = reinterpret_cast<float*>(xs + geo.Z + 1);   // P > 1: the R * P unit sums, 64 per unit
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the table reads are scalar loads
    // workgroup -> (slice, block, index among the workgroups of the pair); consecutive
    // workgroups go to different XCDs, so the workgroups of an XCD share one slice in its L2
    const int s = bid % kSlices;
    const int rest = bid / kSlices;
    const int k = rest % geo.J, wi = rest / geo.J;
    const int out_pad = geo.n_rt * 64;

    // units (r, p) of this workgroup: its r-th row tile, p-th of P equal parts of the steps
    const int n_units = geo.R * geo.P;
    struct Work {
        const uint32_t* e;   // this lane's column of the unit's entries
        int t0, n, rt;       // first step, steps, row tile (rt < 0: no unit)
    };
    auto work_of = [&](int uu) -> Work {
        Work w{entries, 0, 0, -1};
        if (uu >= n_units) return w;
        const int r = uu / geo.P, p = uu % geo.P;
        const int rt = wi + r * geo.W;
        if (rt >= geo.n_rt) return w;
        const int64_t unit = ((int64_t)s * geo.J + k) * geo.n_rt + rt;
        const uint64_t off = table[2 * unit];
        uint64_t L = table[2 * unit + 1];
        if (off + L > cap_steps) L = 0;   // a table that does not fit the entries reads nothing
        w.t0 = (int)((uint64_t)p * L / geo.P);
        w.n = (int)((uint64_t)(p + 1) * L / geo.P) - w.t0;
        w.e = entries + off * 64 + lane;
        w.rt = rt;
        return w;
    };
    // step t of a unit's part, clamped to its last step (prefetches past the end reread it)
    auto fetch = [&](const Work& w, int t) -> uint32_t { return w.e[(size_t)(w.t0 + min(t, w.n - 1)) * 64]; };
    auto lookup = [&](uint32_t en, float acc) {
        return dot8(cbs[en & (kSliceWords - 1)], xs[min((int)(en >> kSliceBits), geo.Z)], acc);
    };
    auto finish = [&](const Work& w, int uu, float acc) {
        if (geo.P > 1)
            red[uu * 64 + lane] = acc;
        else
            partial[(size_t)(s * geo.J + k) * out_pad + w.rt * 64 + lane] = acc;
    };
    uint32_t ra[RING] = {}, rb[RING] = {};
    // Short parts: one ring of RING entries, refilled a chunk ahead.  Every chunk
    // issues its 2 RING LDS reads before the first product.
    auto run_short = [&](const Work& w, int uu) {
        float acc = 0.f;
        int base = 0;
        for (; base + RING <= w.n; base += RING) {
            u32x4 wv[RING], xv[RING];
#pragma unroll
            for (int i = 0; i < RING; ++i) {
                const uint32_t en = ra[i];
                ra[i] = fetch(w, base + i + RING);
                wv[i] = cbs[en & (kSliceWords - 1)];
                xv[i] = xs[min((int)(en >> kSliceBits), geo.Z)];
            }
#pragma unroll
            for (int i = 0; i < RING; ++i) acc = dot8(wv[i], xv[i], acc);
        }
#pragma unroll
        for (int i = 0; i < RING; ++i)   // the last n % RING steps, in order
            if (base + i < w.n) acc = lookup(ra[i], acc);
        finish(w, uu, acc);
    };
    // Long parts: two rings; chunk c is consumed from ring c % 2 while the other ring is
    // in flight, so a chunk waits only for loads issued a whole chunk earlier.
    auto run_long = [&](const Work& w, int uu) {
        float acc = 0.f;
        auto chunk = [&](uint32_t(&r)[RING], int next) {
            u32x4 wv[RING], xv[RING];
#pragma unroll
            for (int i = 0; i < RING; ++i) {
                wv[i] = cbs[r[i] & (kSliceWords - 1)];
                xv[i] = xs[min((int)(r[i] >> kSliceBits), geo.Z)];
            }
#pragma unroll
            for (int i = 0; i < RING; ++i) r[i] = fetch(w, next + i);
#pragma unroll
            for (int i = 0; i < RING; ++i) acc = dot8(wv[i], xv[i], acc);
        };
        int base = 0;
        for (; base + 2 * RING <= w.n; base += 2 * RING) {
            chunk(ra, base + 2 * RING);
            __builtin_amdgcn_sched_barrier(0);   // keep ring a's refill ahead of ring b's reads
            chunk(rb, base + 3 * RING);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < RING; ++i)   // the last n % (2 RING) steps, in order
            if (base + i < w.n) acc = lookup(ra[i], acc);
#pragma unroll
        for (int i = 0; i < RING; ++i)
            if (base + RING + i < w.n) acc = lookup(rb[i], acc);
        finish(w, uu, acc);
    };
    auto prefetch_long = [&](const Work& w) {
#pragma unroll
        for (int i = 0; i < RING; ++i) ra[i] = fetch(w, i);
#pragma unroll
        for (int i = 0; i < RING; ++i) rb[i] = fetch(w, RING + i);
    };

    // the wave's first unit: its table entry (a scalar load) is read before the LDS fill,
    // and its first entries are requested right after the fill, so that they arrive while
    // the fill is in flight without delaying it
    const Work first = work_of(wave);

    // slice and x block into LDS (lane l of a wave writes 16 bytes at base + 16 l)
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(codebook) + (size_t)s * kSliceWords;
#pragma unroll
        for (int i = 0; i < kSliceWords / kListThreads; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(src + i * kListThreads + tid),
                                             lds_ptr(cbs + i * kListThreads + wave * 64), 16, 0, 0);
        const int j0 = k * geo.Gb;
        const int nk = min(geo.G - j0, geo.Gb);   // chunks of this block; whole waves of 64 are copied
        const u32x4* xsrc = reinterpret_cast<const u32x4*>(x) + j0;
        if (wave * 64 < nk)
            __builtin_amdgcn_global_load_lds((const void*)(xsrc + min(tid, nk - 1)), lds_ptr(xs + wave * 64), 16, 0,
                                             0);
        if (tid == 0) xs[geo.Z] = u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (LONG) {
        if (first.n > 0) prefetch_long(first);
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
        __builtin_amdgcn_s_barrier();
        if (first.rt >= 0) run_long(first, wave);
        for (int uu = wave + kListWaves; uu < n_units; uu += kListWaves) {   // only when R > 16 (then P = 1)
            const Work w = work_of(uu);
            if (w.rt < 0) break;
            if (w.n > 0) prefetch_long(w);
            run_long(w, uu);
        }
    } else {
        // Exactly RING vector loads follow the fill: once at most RING loads are
        // pending, this wave's part of the fill has landed (loads complete in order).  A wave
        // without steps reads one of the table's first two words instead; both addresses
        // depend on the lane, so neither can become a scalar load.
        const bool any = first.n > 0;
        const uint32_t* stand_in = table + (lane & 1);
#pragma unroll
        for (int i = 0; i < RING; ++i)
            ra[i] = *(any ? first.e + (size_t)(first.t0 + min(i, first.n - 1)) * 64 : stand_in);
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(RING));
        __builtin_amdgcn_s_barrier();
        if (first.rt >= 0) run_short(first, wave);
        for (int uu = wave + kListWaves; uu < n_units; uu += kListWaves) {
            const Work w = work_of(uu);
            if (w.rt < 0) break;
            if (w.n > 0) {
#pragma unroll
                for (int i = 0; i < RING; ++i) ra[i] = fetch(w, i);
            }
            run_short(w, uu);
        }
    }
    if (geo.P > 1) {   // R * P <= 16: each wave had at most one unit; wave r adds the P parts of row tile r
        __syncthreads();
        const int rt = wi + wave * geo.W;
        if (wave < geo.R && rt < geo.n_rt) {
            float acc = red[wave * geo.P * 64 + lane];
            for (int p = 1; p < geo.P; ++p) acc += red[(wave * geo.P + p) * 64 + lane];
            partial[(size_t)(s * geo.J + k) * out_pad + rt * 64 + lane] = acc;
        }
    }
}

// A single layer: its arguments directly (one small argument block).
template <bool LONG, int RING>
__global__ __launch_bounds__(kListThreads) void gemv_lists_kernel(const uint32_t* __restrict__ table,
                                                                  const uint32_t* __restrict__ entries,
                                                                  uint64_t cap_steps, const f16* __restrict__ codebook,
                                                                  const f16* __restrict__ x,
                                                                  float* __restrict__ partial, ListsGeo geo) {
    lists_product<LONG, RING>(table, entries, cap_steps, codebook, x, partial, geo, blockIdx.x);
}

// Several layers that share x: the workgroup's layer from the table.
template <bool LONG, int RING>
__global__ __launch_bounds__(kListThreads) void gemv_lists_fused_kernel(const ListsLayers L,
                                                                        const f16* __restrict__ x) {
    int first = 0;
    const int l = layer_of(L.wg_end, L.n, blockIdx.x, &first);
    lists_product<LONG, RING>(L.table[l], L.entries[l], L.cap[l], static_cast<const f16*>(L.codebook[l]), x, L.partial[l],
                  L.geo[l], blockIdx.x - first);
}

// y[r] = fp16(s[r] * sum of the row's partials), the slots split into kReduceParts
// contiguous runs added in slot order, then the runs in order.
__device__ __forceinline__ void lists_reduce(const float* __restrict__ partial, const f16* __restrict__ scales,
                                             f16* __restrict__ y, int out, int out_pad, int slots, int blk) {
    __shared__ float red[kReduceParts][64];
    const int rl = threadIdx.x & 63, part = threadIdx.x >> 6;
    const int r = blk * 64 + rl;
    const int per = (slots + kReduceParts - 1) / kReduceParts;
    const int q0 = min(slots, part * per), q1 = min(slots, q0 + per);
    float sum = 0.f;
    if (r < out) {
        for (int qb = q0; qb < q1; qb += 16) {
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = qb + i < q1 ? partial[(size_t)(qb + i) * out_pad + r] : 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) sum += v[i];
        }
    }
    red[part][rl] = sum;
    __syncthreads();
    if (part == 0 && r < out) {
        float t = red[0][rl];
#pragma unroll
        for (int q = 1; q < kReduceParts; ++q) t += red[q][rl];
        y[r] = (f16)(t * (float)scales[r]);
    }
}

__global__ __launch_bounds__(64 * kReduceParts) void lists_reduce_kernel(const float* __restrict__ partial,
                                                                         const f16* __restrict__ scales,
                                                                         f16* __restrict__ y, int out, int out_pad,
                                                                         int slots) {
    lists_reduce(partial, scales, y, out, out_pad, slots, blockIdx.x);
}

__global__ __launch_bounds__(64 * kReduceParts) void lists_reduce_fused_kernel(const ListsLayers L) {
    int first = 0;
    const int l = layer_of(L.blk_end, L.n, blockIdx.x, &first);
    lists_reduce(L.partial[l], static_cast<const f16*>(L.scales[l]), static_cast<f16*>(L.y[l]), L.out[l],
                 L.geo[l].n_rt * 64, L.geo[l].slots(), blockIdx.x - first);
}

}  // namespace

ListsGeo lists_geo(int64_t out, int64_t in) {
    ListsGeo g;
    g.G = (int)(in / 8);
    g.J = (g.G + kListsMaxBlock - 1) / kListsMaxBlock;
    g.Gb = (g.G + g.J - 1) / g.J;
    g.Z = (g.Gb + 63) / 64 * 64;
    g.n_rt = (int)((out + 63) / 64);
    g.W = std::max(1, std::min(kWgPerSlice / g.J, g.n_rt));
    g.R = (g.n_rt + g.W - 1) / g.W;
    g.P = g.R > 0 ? std::max(1, kListWaves / g.R) : 1;   // out == 0: no row tiles
    return g;
}

int64_t lists_table_bytes(int64_t out, int64_t in) {
    const ListsGeo g = lists_geo(out, in);
    return (2 * g.n_units() + 2) * 4;
}

int64_t lists_workspace_bytes(int64_t out, int64_t in) {
    const ListsGeo g = lists_geo(out, in);
    return (int64_t)g.slots() * g.n_rt * 64 * 4;
}

hipError_t launch_lists_plan(const void* codes, int64_t out, int64_t in, void* table, hipStream_t stream) {
    const ListsGeo g = lists_geo(out, in);
    const int64_t blocks = (g.n_units() + 3) / 4;
    if (blocks > 0)
        hipLaunchKernelGGL(lists_count_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(codes), (int)out, g, static_cast<uint32_t*>(table));
    hipLaunchKernelGGL(lists_scan_kernel, dim3(1), dim3(1024), 0, stream, g, static_cast<uint32_t*>(table));
    return hipGetLastError();
}

hipError_t launch_lists_fill(const void* codes, int64_t out, int64_t in, const void* table, void* entries,
                             int64_t entries_bytes, hipStream_t stream) {
    const ListsGeo g = lists_geo(out, in);
    const int64_t blocks = (g.n_units() + 3) / 4;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(lists_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(codes), (int)out, g, static_cast<const uint32_t*>(table),
                       static_cast<uint32_t*>(entries), (uint64_t)(entries_bytes / 256));
    return hipGetLastError();
}

int64_t lists_workspace_bytes_aligned(int64_t out, int64_t in) {
    return (lists_workspace_bytes(out, in) + 255) / 256 * 256;
}

// The caller has filled every per-layer field but geo, wg_end and blk_end (out > 0 for every layer).
hipError_t launch_gemv_lists_fused(ListsLayers L, const void* x, int64_t in, hipStream_t stream) {
    size_t lds = 0;
    int64_t wgs = 0, blks = 0;
    for (int l = 0; l < L.n; ++l) {
        const ListsGeo g = lists_geo(L.out[l], in);
        L.geo[l] = g;
        lds = std::max(lds, (size_t)kSliceWords * 16 + (size_t)(g.Z + 1) * 16 +
                                (g.P > 1 ? (size_t)g.R * g.P * 64 * 4 : 0));
        wgs += (int64_t)kSlices * g.J * g.W;
        blks += (L.out[l] + 63) / 64;
        if (wgs > INT32_MAX || blks > INT32_MAX) return hipErrorInvalidValue;
        L.wg_end[l] = (int)wgs;
        L.blk_end[l] = (int)blks;
    }
    const bool multi = L.n > 1;
    // long parts: about Gb/8 steps per row tile (uniform codes) split over P waves
    bool long_parts = true;
    for (int l = 0; l < L.n; ++l) long_parts &= L.geo[l].Gb / 8 / L.geo[l].P >= kListLongPart;
    // one-ring launches whose every wave has a unit keep fewer entry loads in flight: measured
    // 2-4 % faster on such layers (4096^2, 8192^2, 4096x11008) and 6 % slower where waves idle
    bool busy = !long_parts;
    for (int l = 0; l < L.n; ++l) busy &= (int64_t)L.geo[l].R * L.geo[l].P >= kListWaves;
    auto fk = long_parts ? gemv_lists_fused_kernel<true, kListRing>
                         : (busy ? gemv_lists_fused_kernel<false, kListRingBusy> : gemv_lists_fused_kernel<false, kListRing>);
    auto sk = long_parts ? gemv_lists_kernel<true, kListRing>
                         : (busy ? gemv_lists_kernel<false, kListRingBusy> : gemv_lists_kernel<false, kListRing>);
    const void* kern = multi ? (const void*)fk : (const void*)sk;
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (multi) {
        hipLaunchKernelGGL(fk, dim3((unsigned)wgs), dim3(kListThreads), lds, stream, L, static_cast<const f16*>(x));
        hipLaunchKernelGGL(lists_reduce_fused_kernel, dim3((unsigned)blks), dim3(64 * kReduceParts), 0, stream, L);
    } else {   // one layer: the compact argument lists
        const ListsGeo& g = L.geo[0];
        hipLaunchKernelGGL(sk, dim3((unsigned)wgs), dim3(kListThreads), lds, stream, L.table[0],
                           L.entries[0], L.cap[0], static_cast<const f16*>(L.codebook[0]),
                           static_cast<const f16*>(x), L.partial[0], g);
        hipLaunchKernelGGL(lists_reduce_kernel, dim3((unsigned)blks), dim3(64 * kReduceParts), 0, stream,
                           static_cast<const float*>(L.partial[0]), static_cast<const f16*>(L.scales[0]),
                           static_cast<f16*>(L.y[0]), L.out[0], g.n_rt * 64, g.slots());
    }
    return hipGetLastError();
}

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t lists_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with this device current
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_gemv_lists(const void* table, const void* entries, int64_t entries_bytes, const void* codebook,
                             const void* scales, const void* x, void* y, void* workspace, int64_t out, int64_t in,
                             hipStream_t stream) {
    ListsLayers L{};
    L.n = 1;
    L.table[0] = static_cast<const uint32_t*>(table);
    L.entries[0] = static_cast<const uint32_t*>(entries);
    L.cap[0] = (uint64_t)(entries_bytes / 256);
    L.codebook[0] = codebook;
    L.scales[0] = scales;
    L.y[0] = y;
    L.partial[0] = static_cast<float*>(workspace);
    L.out[0] = (int)out;
    return launch_gemv_lists_fused(L, x, in, stream);
}

}  // namespace aqlm
