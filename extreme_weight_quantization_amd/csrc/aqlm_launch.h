// Host-side launchers of the AQLM kernels (called by the C ABI in aqlm_api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aqlm {

// Compute units of the current device (cached per device).
int device_cu_count();

// A scheme other than 1x16 and 2x8 at g = 8: 1 <= M <= 8, 1 <= B <= 16,
// g in {1, 2, 4, 8, 16, 32}; codes are uint8 for B <= 8, else 16-bit.
// packed: the codes are one bit stream (code n in bits [n B, n B + B) of little-endian
// 32-bit words, least significant bit first) instead of whole bytes per code.
struct GenericScheme {
    int M, B, g;
    bool packed = false;
};
// 32-bit words of the bit-packed codes of a layer, and the packing kernel (from the
// whole-byte codes [out][in/g][M]).
uint64_t packed_code_words(int M, int B, int g, int64_t out, int64_t in);
hipError_t launch_pack_codes(const void* codes, void* words, int M, int B, int g, int64_t out, int64_t in,
                             hipStream_t stream);

hipError_t launch_decode_generic(const GenericScheme& sc, const void* codes, const void* codebooks,
                                 const void* scales, void* w, int64_t out, int64_t in, hipStream_t stream);
hipError_t launch_gemv_generic(const GenericScheme& sc, const void* codes, const void* codebooks,
                               const void* scales, const void* x, void* y, int64_t out, int64_t in,
                               int64_t batch, hipStream_t stream);
// Greedy residual codes with fixed codebooks, and residual k-means (encode.hip).
hipError_t launch_encode_greedy(const void* w, const void* scales, const void* codebooks, void* codes, int M, int B,
                                int g, int64_t out, int64_t in, hipStream_t stream);
hipError_t launch_kmeans_init(const void* w, const void* scales, const int64_t* seeds, void* codebooks, void* codes,
                              void* workspace, int M, int B, int g, int64_t out, int64_t in, int iters,
                              hipStream_t stream);
int64_t kmeans_workspace_bytes(int M, int B, int g);

hipError_t launch_gemm_generic(const GenericScheme& sc, const void* codes, const void* codebooks,
                               const void* scales, const void* x, void* y, int64_t out, int64_t in,
                               int64_t batch, hipStream_t stream);

hipError_t launch_decode(int scheme, const void* codes, const void* codebooks, const void* scales,
                         void* w, int64_t out, int64_t in, hipStream_t stream);

// Layers of one GEMV launch: every layer has its own codes, codebooks, scales,
// y and out, and all of them share x, in, batch and the scheme.  Workgroups
// [wg_end[l-1], wg_end[l]) serve layer l (wg_end[-1] = 0); the launcher fills
// wg_end.  Passed to the kernel by value.
constexpr int kGemvMaxLayers = 8;
struct GemvLayers {
    const void* codes[kGemvMaxLayers];
    const void* codebooks[kGemvMaxLayers];
    const void* scales[kGemvMaxLayers];
    void* y[kGemvMaxLayers];
    int out[kGemvMaxLayers];
    int wg_end[kGemvMaxLayers];
    int n;
};

// Several layers that share x in one launch (layers with out == 0 must be left out).
hipError_t launch_gemv_fused(int scheme, GemvLayers layers, const void* x, int64_t in,
                             int64_t batch, hipStream_t stream);

hipError_t launch_gemv(int scheme, const void* codes, const void* codebooks, const void* scales,
                       const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                       hipStream_t stream);

// The streaming 2x8 product for batch 1-4 (gemv_stream.hip).  gemv_stream_lds: its LDS
// bytes for layers whose workgroups are dealt, or 0 where it does not serve them.
size_t gemv_stream_lds(const GemvLayers& layers, int64_t in, int64_t batch);
hipError_t launch_gemv_stream(const GemvLayers& layers, const void* x, int64_t in, int64_t batch, size_t lds,
                              hipStream_t stream);

// 2x8 prefill product with the role-split pipeline; requires in % 64 == 0.
hipError_t launch_gemm_pipe_2x8(const void* codes, const void* codebooks, const void* scales,
                                const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                                hipStream_t stream);
// The same pipeline for 1x8 g4 (its codes also take 2 bytes per 8 inputs); in % 64 == 0.
hipError_t launch_gemm_pipe_1x8g4(const void* codes, const void* codebooks, const void* scales,
                                  const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                                  hipStream_t stream);
// And for 1x16 (16-bit codes, codewords gathered from L2 by producer waves of their own); in % 64 == 0.
hipError_t launch_gemm_pipe_1x16(const void* codes, const void* codebooks, const void* scales,
                                 const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                                 hipStream_t stream);
// And for 4x8 g16 (4 code bytes per 16 inputs, also 2 bytes per 8 at the same places); in % 64 == 0.
hipError_t launch_gemm_pipe_4x8g16(const void* codes, const void* codebooks, const void* scales,
                                   const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                                   hipStream_t stream);

// Dense fp16 product y[t][i] = sum_k x[t][k] w16[i][k] (gemm_dense.hip); requires in % 64 == 0.
hipError_t launch_gemm_dense(const void* x, const void* w16, void* y, int64_t out, int64_t in, int64_t batch,
                             hipStream_t stream);

hipError_t launch_gemm(int scheme, const void* codes, const void* codebooks, const void* scales,
                       const void* x, void* y, int64_t out, int64_t in, int64_t batch,
                       hipStream_t stream);

// 1x16 products over slice lists (gemv_lists.hip): codes regrouped by codebook
// slice per 64-row tile and per block of at most kListsMaxBlock groups.  The
// geometry depends on (out, in) only.
constexpr int kListsMaxBlock = 1024;
struct ListsGeo {
    int G;      // groups per row (in / 8)
    int J;      // blocks of groups
    int Gb;     // groups per block (the last may have fewer)
    int Z;      // Gb rounded up to 64: index of the zero x chunk that padding entries name
    int n_rt;   // 64-row tiles
    int W;      // workgroups per (slice, block)
    int R;      // row tiles per workgroup (at most)
    int P;      // parts the steps of a unit are split into
    __host__ __device__ int64_t n_units() const { return (int64_t)8 * J * n_rt; }
    __host__ __device__ int slots() const { return 8 * J; }   // partial sums per row
};
ListsGeo lists_geo(int64_t out, int64_t in);

// Layers of one slice-list product launch: all share x and in; layer l has its
// own table, entries (cap = entries_bytes / 256 steps), codebook, scales, y,
// partial sums (fp32, 8 J * 64 n_rt) and geometry.  Product workgroups
// [wg_end[l-1], wg_end[l]) and reduction blocks [blk_end[l-1], blk_end[l])
// serve layer l; the launcher fills both.  Passed to the kernels by value.
struct ListsLayers {
    const uint32_t* table[kGemvMaxLayers];
    const uint32_t* entries[kGemvMaxLayers];
    uint64_t cap[kGemvMaxLayers];
    const void* codebook[kGemvMaxLayers];
    const void* scales[kGemvMaxLayers];
    void* y[kGemvMaxLayers];
    float* partial[kGemvMaxLayers];
    ListsGeo geo[kGemvMaxLayers];
    int out[kGemvMaxLayers];
    int wg_end[kGemvMaxLayers];
    int blk_end[kGemvMaxLayers];
    int n;
};
// Bytes of fp32 partial sums of one layer, rounded up to 256 (a fused launch
// places the layers' partials one after another in its workspace).
int64_t lists_workspace_bytes_aligned(int64_t out, int64_t in);
hipError_t launch_gemv_lists_fused(ListsLayers layers, const void* x, int64_t in, hipStream_t stream);
int64_t lists_table_bytes(int64_t out, int64_t in);
int64_t lists_workspace_bytes(int64_t out, int64_t in);
hipError_t launch_lists_plan(const void* codes, int64_t out, int64_t in, void* table, hipStream_t stream);
hipError_t launch_lists_fill(const void* codes, int64_t out, int64_t in, const void* table, void* entries,
                             int64_t entries_bytes, hipStream_t stream);
hipError_t launch_gemv_lists(const void* table, const void* entries, int64_t entries_bytes, const void* codebook,
                             const void* scales, const void* x, void* y, void* workspace, int64_t out, int64_t in,
                             hipStream_t stream);
// Bytes of the static scratch array of the allocation-free slice-list product.
constexpr int64_t kListsScratchBytes = (int64_t)4 << 20;
// This device's address of that array (looked up once per device; thread-safe).
hipError_t lists_scratch(void** ptr);

}  // namespace aqlm
