// C ABI of libaqlm.so (declared in include/aqlm.h): argument validation on the
// host, then dispatch to the HIP kernels on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/aqlm.h"
#include "aqlm_device.h"
#include "aqlm_launch.h"

static_assert(AQLM_FUSED_MAX_LAYERS == aqlm::kGemvMaxLayers, "fused layer limit");

namespace aqlm {

namespace {
thread_local int g_last_hip_error = 0;
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
}  // namespace

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

enum class Op { kGemv, kGemm, kDecode };

static bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static bool generic_scheme_ok(int M, int B, int g) {
    return M >= 1 && M <= AQLM_MAX_CODEBOOKS && B >= 1 && B <= 16 &&
           (g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32);
}

// The GEMV of the other 2-bit schemes with B = 8 (g = 4 M) runs the 2x8 product's
// kernel, which reads 2 bytes of codes per 8 inputs (in % 8 == 0): 1x8 g4 and 4x8 g16
// at every batch, 8x8 g32 above batch 8 (below, where its eight lookups per 8 inputs
// and single codebook copy dominate, the general kernel was faster).  -1: the
// general kernel.
static int gemv_b8_scheme(int M, int B, int g, int64_t in, int64_t batch) {
    if (B != 8 || g != 4 * M || in % 8 != 0) return -1;
    if (M == 1) return kSchemeB8M1;
    if (M == 4) return kSchemeB8M4;
    if (M == 8 && batch > 8) return kSchemeB8M8;
    return -1;
}

// Host-side validation shared by the entry points.  Returns AQLM_OK and the
// scheme id, or an error status; touches no HIP state.
static int validate(Op op, const void* codes, const void* codebooks, const void* scales,
                    const void* x, const void* y, int M, int B, int g, int64_t out, int64_t in,
                    int64_t batch, int* scheme, bool* empty, uintptr_t codes_align = 16) {
    if (op == Op::kDecode && x != nullptr) return AQLM_ERR_NULL;
    if (M == 1 && B == 16 && g == 8) *scheme = kScheme1x16;
    else if (M == 2 && B == 8 && g == 8) *scheme = kScheme2x8;
    else if (generic_scheme_ok(M, B, g)) *scheme = kSchemeGeneric;
    else return AQLM_ERR_SCHEME;
    if (out < 0 || in < 1 || in > AQLM_MAX_IN || (in % g) != 0) return AQLM_ERR_SHAPE;
    if (out > (int64_t)INT32_MAX - 16) return AQLM_ERR_SHAPE;
    if (op == Op::kGemv && (batch < 0 || batch > AQLM_GEMV_MAX_BATCH)) return AQLM_ERR_SHAPE;
    if (op == Op::kGemm && (batch < 0 || batch > (int64_t)INT32_MAX - 256)) return AQLM_ERR_SHAPE;
    if (op == Op::kDecode && (uint64_t)out * (uint64_t)(in / g) > (uint64_t)UINT32_MAX) return AQLM_ERR_SHAPE;
    if (op == Op::kGemm) {
        const uint64_t tiles = (uint64_t)((out + 127) / 128) * (uint64_t)((batch + 127) / 128);
        if (tiles > (uint64_t)INT32_MAX) return AQLM_ERR_SHAPE;
    }
    // An empty problem reads and writes nothing: its (possibly NULL) pointers are not used.
    *empty = (out == 0) || (op != Op::kDecode && batch == 0);
    if (*empty) return AQLM_OK;
    if (!codes || !codebooks || !scales || !y) return AQLM_ERR_NULL;
    if (op != Op::kDecode && x == nullptr) return AQLM_ERR_NULL;
    if (!aligned(codes, codes_align) || !aligned(codebooks, 16) || !aligned(y, 16) || !aligned(scales, 2))
        return AQLM_ERR_ALIGN;
    if (x && !aligned(x, 16)) return AQLM_ERR_ALIGN;
    return AQLM_OK;
}

static int finish(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return AQLM_ERR_HIP;
    }
    return AQLM_OK;
}

}  // namespace aqlm

using namespace aqlm;

extern "C" {

int aqlm_linear_gemv(const void* codes, const void* codebooks, const void* scales, const void* x,
                     void* y, int M, int B, int g, int64_t out, int64_t in, int64_t batch,
                     void* stream) {
    int scheme = 0;
    bool empty = false;
    const int st = validate(Op::kGemv, codes, codebooks, scales, x, y, M, B, g, out, in, batch, &scheme, &empty);
    if (st != AQLM_OK || empty) return st;
    if (scheme == kSchemeGeneric && gemv_b8_scheme(M, B, g, in, batch) >= 0) scheme = gemv_b8_scheme(M, B, g, in, batch);
    if (scheme == kSchemeGeneric)
        return finish(launch_gemv_generic(GenericScheme{M, B, g}, codes, codebooks, scales, x, y, out, in,
                                          batch, (hipStream_t)stream));
    return finish(launch_gemv(scheme, codes, codebooks, scales, x, y, out, in, batch,
                              (hipStream_t)stream));
}

int aqlm_linear_gemv_fused(int n_layers, const void* const* codes, const void* const* codebooks,
                           const void* const* scales, const int64_t* outs, const void* x,
                           void* const* ys, int M, int B, int g, int64_t in, int64_t batch,
                           void* stream) {
    if (n_layers < 1 || n_layers > AQLM_FUSED_MAX_LAYERS) return AQLM_ERR_SHAPE;
    if (!codes || !codebooks || !scales || !outs || !ys) return AQLM_ERR_NULL;
    GemvLayers layers = {};
    int scheme = 0;
    for (int l = 0; l < n_layers; ++l) {
        bool empty = false;
        const int st = validate(Op::kGemv, codes[l], codebooks[l], scales[l], x, ys[l], M, B, g, outs[l],
                                in, batch, &scheme, &empty);
        if (st != AQLM_OK) return st;
        if (empty) continue;
        layers.codes[layers.n] = codes[l];
        layers.codebooks[layers.n] = codebooks[l];
        layers.scales[layers.n] = scales[l];
        layers.y[layers.n] = ys[l];
        layers.out[layers.n] = (int)outs[l];
        ++layers.n;
    }
    if (layers.n == 0) return AQLM_OK;
    if (scheme == kSchemeGeneric && gemv_b8_scheme(M, B, g, in, batch) >= 0) scheme = gemv_b8_scheme(M, B, g, in, batch);
    if (scheme == kSchemeGeneric) {   // one launch per layer
        for (int l = 0; l < layers.n; ++l) {
            const int st = finish(launch_gemv_generic(GenericScheme{M, B, g}, layers.codes[l], layers.codebooks[l],
                                                      layers.scales[l], x, layers.y[l], layers.out[l], in, batch,
                                                      (hipStream_t)stream));
            if (st != AQLM_OK) return st;
        }
        return AQLM_OK;
    }
    return finish(launch_gemv_fused(scheme, layers, x, in, batch, (hipStream_t)stream));
}

int aqlm_linear_gemm(const void* codes, const void* codebooks, const void* scales, const void* x,
                     void* y, int M, int B, int g, int64_t out, int64_t in, int64_t batch,
                     void* stream) {
    int scheme = 0;
    bool empty = false;
    const int st = validate(Op::kGemm, codes, codebooks, scales, x, y, M, B, g, out, in, batch, &scheme, &empty);
    if (st != AQLM_OK || empty) return st;
    if (M == 1 && B == 8 && g == 4 && in % 64 == 0)   // the 2x8 pipeline with two 4-entry codewords a piece
        return finish(launch_gemm_pipe_1x8g4(codes, codebooks, scales, x, y, out, in, batch, (hipStream_t)stream));
    if (M == 4 && B == 8 && g == 16 && in % 64 == 0)   // the 2x8 pipeline, four 16-entry codewords a group
        return finish(launch_gemm_pipe_4x8g16(codes, codebooks, scales, x, y, out, in, batch, (hipStream_t)stream));
    if (scheme == kSchemeGeneric)
        return finish(launch_gemm_generic(GenericScheme{M, B, g}, codes, codebooks, scales, x, y, out, in,
                                          batch, (hipStream_t)stream));
    return finish(launch_gemm(scheme, codes, codebooks, scales, x, y, out, in, batch,
                              (hipStream_t)stream));
}

// ---- bit-packed codes: every scheme, on the general kernels
int aqlm_packed_codes_bytes(int M, int B, int g, int64_t out, int64_t in, int64_t* bytes) {
    if (!bytes) return AQLM_ERR_NULL;
    if (!generic_scheme_ok(M, B, g)) return AQLM_ERR_SCHEME;
    if (out < 0 || out > (int64_t)INT32_MAX - 16 || in < 1 || in > AQLM_MAX_IN || (in % g) != 0)
        return AQLM_ERR_SHAPE;
    *bytes = (int64_t)packed_code_words(M, B, g, out, in) * 4;
    return AQLM_OK;
}

int aqlm_pack_codes(const void* codes, void* packed, int M, int B, int g, int64_t out, int64_t in, void* stream) {
    if (!generic_scheme_ok(M, B, g)) return AQLM_ERR_SCHEME;
    if (out < 0 || out > (int64_t)INT32_MAX - 16 || in < 1 || in > AQLM_MAX_IN || (in % g) != 0)
        return AQLM_ERR_SHAPE;
    if (out == 0) return AQLM_OK;
    if (!codes || !packed) return AQLM_ERR_NULL;
    if (!aligned(codes, B <= 8 ? 1 : 2) || !aligned(packed, 4)) return AQLM_ERR_ALIGN;
    return finish(launch_pack_codes(codes, packed, M, B, g, out, in, (hipStream_t)stream));
}

static int packed_call(Op op, const void* codes, const void* codebooks, const void* scales, const void* x, void* y,
                       int M, int B, int g, int64_t out, int64_t in, int64_t batch, void* stream) {
    int scheme = 0;
    bool empty = false;
    const int st = validate(op, codes, codebooks, scales, x, y, M, B, g, out, in, batch, &scheme, &empty, 4);
    if (st != AQLM_OK || empty) return st;
    GenericScheme sc{M, B, g};
    sc.packed = true;
    const hipStream_t s = (hipStream_t)stream;
    if (op == Op::kGemv) return finish(launch_gemv_generic(sc, codes, codebooks, scales, x, y, out, in, batch, s));
    if (op == Op::kGemm) return finish(launch_gemm_generic(sc, codes, codebooks, scales, x, y, out, in, batch, s));
    return finish(launch_decode_generic(sc, codes, codebooks, scales, y, out, in, s));
}

int aqlm_linear_gemv_packed(const void* codes, const void* codebooks, const void* scales, const void* x, void* y,
                            int M, int B, int g, int64_t out, int64_t in, int64_t batch, void* stream) {
    return packed_call(Op::kGemv, codes, codebooks, scales, x, y, M, B, g, out, in, batch, stream);
}

int aqlm_linear_gemm_packed(const void* codes, const void* codebooks, const void* scales, const void* x, void* y,
                            int M, int B, int g, int64_t out, int64_t in, int64_t batch, void* stream) {
    return packed_call(Op::kGemm, codes, codebooks, scales, x, y, M, B, g, out, in, batch, stream);
}

int aqlm_linear_decode_packed(const void* codes, const void* codebooks, const void* scales, const void* x, void* y,
                              int M, int B, int g, int64_t out, int64_t in, int64_t batch, void* stream) {
    (void)batch;
    return packed_call(Op::kDecode, codes, codebooks, scales, x, y, M, B, g, out, in, 1, stream);
}

int aqlm_gemm_dequant_workspace_bytes(int M, int B, int g, int64_t out, int64_t in, int64_t* bytes) {
    if (!bytes) return AQLM_ERR_NULL;
    if (!(M == 1 && B == 16 && g == 8) && !(M == 2 && B == 8 && g == 8) && !generic_scheme_ok(M, B, g))
        return AQLM_ERR_SCHEME;
    if (out < 0 || in < 1 || in > AQLM_MAX_IN || (in % g) != 0 || out > (int64_t)INT32_MAX - 16)
        return AQLM_ERR_SHAPE;
    *bytes = (in % 64 == 0) ? out * in * 2 : 0;
    return AQLM_OK;
}

int aqlm_linear_gemm_dequant(const void* codes, const void* codebooks, const void* scales, const void* x,
                             void* y, void* workspace, int64_t workspace_bytes, int M, int B, int g, int64_t out,
                             int64_t in, int64_t batch, void* stream) {
    int scheme = 0;
    bool empty = false;
    const int st = validate(Op::kGemm, codes, codebooks, scales, x, y, M, B, g, out, in, batch, &scheme, &empty);
    if (st != AQLM_OK) return st;
    if ((uint64_t)out * (uint64_t)(in / g) > (uint64_t)UINT32_MAX) return AQLM_ERR_SHAPE;
    if (empty) return AQLM_OK;
    if (in % 64 != 0)
        return aqlm_linear_gemm(codes, codebooks, scales, x, y, M, B, g, out, in, batch, stream);
    if (!workspace) return AQLM_ERR_NULL;
    if (!aligned(workspace, 16)) return AQLM_ERR_ALIGN;
    if (workspace_bytes < out * in * 2) return AQLM_ERR_SHAPE;
    const hipStream_t s = (hipStream_t)stream;
    const int dst = (scheme == kSchemeGeneric)
                        ? finish(launch_decode_generic(GenericScheme{M, B, g}, codes, codebooks, scales, workspace,
                                                       out, in, s))
                        : finish(launch_decode(scheme, codes, codebooks, scales, workspace, out, in, s));
    if (dst != AQLM_OK) return dst;
    return finish(launch_gemm_dense(x, workspace, y, out, in, batch, s));
}

int aqlm_linear_decode(const void* codes, const void* codebooks, const void* scales, const void* x,
                       void* y, int M, int B, int g, int64_t out, int64_t in, int64_t batch,
                       void* stream) {
    (void)batch;
    int scheme = 0;
    bool empty = false;
    const int st = validate(Op::kDecode, codes, codebooks, scales, x, y, M, B, g, out, in, 1, &scheme, &empty);
    if (st != AQLM_OK || empty) return st;
    if (scheme == kSchemeGeneric)
        return finish(launch_decode_generic(GenericScheme{M, B, g}, codes, codebooks, scales, y, out, in,
                                            (hipStream_t)stream));
    return finish(launch_decode(scheme, codes, codebooks, scales, y, out, in, (hipStream_t)stream));
}

// Shared checks of the encoder entry points (scheme, shape, pointers, alignment).
static int validate_encode(const void* w, const void* scales, const void* codebooks, const void* codes, int M, int B,
                           int g, int64_t out, int64_t in, bool* empty) {
    if (!generic_scheme_ok(M, B, g)) return AQLM_ERR_SCHEME;
    if (out < 0 || out > (int64_t)INT32_MAX || in < 1 || in > AQLM_MAX_IN || (in % g) != 0) return AQLM_ERR_SHAPE;
    *empty = out == 0;
    if (*empty) return AQLM_OK;
    if (!w || !scales || !codebooks || !codes) return AQLM_ERR_NULL;
    if (!aligned(w, 16) || !aligned(codebooks, 16) || !aligned(codes, 16) || !aligned(scales, 2)) return AQLM_ERR_ALIGN;
    return AQLM_OK;
}

int aqlm_encode_greedy(const void* w, const void* scales, const void* codebooks, void* codes, int M, int B, int g,
                       int64_t out, int64_t in, void* stream) {
    bool empty = false;
    const int st = validate_encode(w, scales, codebooks, codes, M, B, g, out, in, &empty);
    if (st != AQLM_OK || empty) return st;
    return finish(launch_encode_greedy(w, scales, codebooks, codes, M, B, g, out, in, (hipStream_t)stream));
}

int aqlm_kmeans_workspace_bytes(int M, int B, int g, int64_t* bytes) {
    if (!bytes) return AQLM_ERR_NULL;
    if (!generic_scheme_ok(M, B, g)) return AQLM_ERR_SCHEME;
    *bytes = kmeans_workspace_bytes(M, B, g);
    return AQLM_OK;
}

int aqlm_kmeans_init(const void* w, const void* scales, const int64_t* seeds, void* codebooks, void* codes,
                     void* workspace, int64_t workspace_bytes, int M, int B, int g, int64_t out, int64_t in,
                     int iters, void* stream) {
    bool empty = false;
    int st = validate_encode(w, scales, codebooks, codes, M, B, g, out, in, &empty);
    if (st != AQLM_OK) return st;
    if (iters < 0 || iters > AQLM_KMEANS_MAX_ITERS) return AQLM_ERR_SHAPE;
    if (empty) return AQLM_OK;
    if (!seeds || !workspace) return AQLM_ERR_NULL;
    if (!aligned(seeds, 8) || !aligned(workspace, 16)) return AQLM_ERR_ALIGN;
    if (workspace_bytes < kmeans_workspace_bytes(M, B, g)) return AQLM_ERR_SHAPE;
    return finish(launch_kmeans_init(w, scales, seeds, codebooks, codes, workspace, M, B, g, out, in, iters,
                                     (hipStream_t)stream));
}

// ---- 1x16 slice lists
static int validate_lists(int M, int B, int g, int64_t out, int64_t in) {
    if (!(M == 1 && B == 16 && g == 8)) return AQLM_ERR_SCHEME;
    if (out < 0 || out > AQLM_LISTS_MAX_OUT || in < 8 || in > AQLM_MAX_IN || (in % 8) != 0) return AQLM_ERR_SHAPE;
    if ((uint64_t)out * (uint64_t)(in / 8) > (uint64_t)UINT32_MAX) return AQLM_ERR_SHAPE;
    return AQLM_OK;
}

int aqlm_lists_table_bytes(int M, int B, int g, int64_t out, int64_t in, int64_t* bytes) {
    if (!bytes) return AQLM_ERR_NULL;
    const int st = validate_lists(M, B, g, out, in);
    if (st != AQLM_OK) return st;
    *bytes = lists_table_bytes(out, in);
    return AQLM_OK;
}

int aqlm_lists_workspace_bytes(int M, int B, int g, int64_t out, int64_t in, int64_t* bytes) {
    if (!bytes) return AQLM_ERR_NULL;
    const int st = validate_lists(M, B, g, out, in);
    if (st != AQLM_OK) return st;
    *bytes = lists_workspace_bytes(out, in);
    return AQLM_OK;
}

int aqlm_lists_plan(const void* codes, void* table, int M, int B, int g, int64_t out, int64_t in, void* stream) {
    const int st = validate_lists(M, B, g, out, in);
    if (st != AQLM_OK) return st;
    if (!table || (out > 0 && !codes)) return AQLM_ERR_NULL;
    if (!aligned(table, 16) || (codes && !aligned(codes, 16))) return AQLM_ERR_ALIGN;
    return finish(launch_lists_plan(codes, out, in, table, (hipStream_t)stream));
}

int aqlm_lists_fill(const void* codes, const void* table, void* entries, int64_t entries_bytes, int M, int B, int g,
                    int64_t out, int64_t in, void* stream) {
    const int st = validate_lists(M, B, g, out, in);
    if (st != AQLM_OK) return st;
    if (entries_bytes < 0) return AQLM_ERR_SHAPE;
    if (out == 0) return AQLM_OK;
    if (!codes || !table || !entries) return AQLM_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(table, 16) || !aligned(entries, 16)) return AQLM_ERR_ALIGN;
    return finish(launch_lists_fill(codes, out, in, table, entries, entries_bytes, (hipStream_t)stream));
}

int aqlm_linear_gemv_lists(const void* table, const void* entries, int64_t entries_bytes, const void* codebooks,
                           const void* scales, const void* x, void* y, void* workspace, int64_t workspace_bytes, int M,
                           int B, int g, int64_t out, int64_t in, int64_t batch, void* stream) {
    const int st = validate_lists(M, B, g, out, in);
    if (st != AQLM_OK) return st;
    if (batch < 0 || batch > 1 || entries_bytes < 0 || workspace_bytes < 0) return AQLM_ERR_SHAPE;
    if (out == 0 || batch == 0) return AQLM_OK;
    if (!table || !entries || !codebooks || !scales || !x || !y || !workspace) return AQLM_ERR_NULL;
    if (!aligned(table, 16) || !aligned(entries, 16) || !aligned(codebooks, 16) || !aligned(x, 16) ||
        !aligned(y, 16) || !aligned(workspace, 16) || !aligned(scales, 2))
        return AQLM_ERR_ALIGN;
    if (workspace_bytes < lists_workspace_bytes(out, in)) return AQLM_ERR_SHAPE;
    return finish(launch_gemv_lists(table, entries, entries_bytes, codebooks, scales, x, y, workspace, out, in,
                                    (hipStream_t)stream));
}

static_assert(AQLM_LISTS_NOALLOC_SCRATCH_BYTES == kListsScratchBytes, "scratch size");

int aqlm_linear_gemv_lists_noalloc(const void* table, const void* entries, int64_t entries_bytes,
                                   const void* codebooks, const void* scales, const void* x, void* y, int M, int B,
                                   int g, int64_t out, int64_t in, int64_t batch, void* stream) {
    const int st = validate_lists(M, B, g, out, in);
    if (st != AQLM_OK) return st;
    if (batch < 0 || batch > 1 || entries_bytes < 0) return AQLM_ERR_SHAPE;
    if (lists_workspace_bytes(out, in) > kListsScratchBytes) return AQLM_ERR_SCRATCH;
    if (out == 0 || batch == 0) return AQLM_OK;
    if (!table || !entries || !codebooks || !scales || !x || !y) return AQLM_ERR_NULL;
    if (!aligned(table, 16) || !aligned(entries, 16) || !aligned(codebooks, 16) || !aligned(x, 16) ||
        !aligned(y, 16) || !aligned(scales, 2))
        return AQLM_ERR_ALIGN;
    void* partial = nullptr;
    const hipError_t e = lists_scratch(&partial);
    if (e != hipSuccess) return finish(e);
    return finish(launch_gemv_lists(table, entries, entries_bytes, codebooks, scales, x, y, partial, out, in,
                                    (hipStream_t)stream));
}

int aqlm_lists_fused_workspace_bytes(int n_layers, const int64_t* outs, int M, int B, int g, int64_t in,
                                     int64_t* bytes) {
    if (!bytes || !outs) return AQLM_ERR_NULL;
    if (n_layers < 1 || n_layers > AQLM_FUSED_MAX_LAYERS) return AQLM_ERR_SHAPE;
    int64_t total = 0;
    for (int l = 0; l < n_layers; ++l) {
        const int st = validate_lists(M, B, g, outs[l], in);
        if (st != AQLM_OK) return st;
        if (outs[l] > 0) total += lists_workspace_bytes_aligned(outs[l], in);
    }
    *bytes = total;
    return AQLM_OK;
}

int aqlm_linear_gemv_lists_fused(int n_layers, const void* const* tables, const void* const* entries,
                                 const int64_t* entries_bytes, const void* const* codebooks, const void* const* scales,
                                 const int64_t* outs, const void* x, void* const* ys, void* workspace,
                                 int64_t workspace_bytes, int M, int B, int g, int64_t in, int64_t batch,
                                 void* stream) {
    if (n_layers < 1 || n_layers > AQLM_FUSED_MAX_LAYERS) return AQLM_ERR_SHAPE;
    if (!tables || !entries || !entries_bytes || !codebooks || !scales || !outs || !ys) return AQLM_ERR_NULL;
    if (batch < 0 || batch > 1 || workspace_bytes < 0) return AQLM_ERR_SHAPE;
    ListsLayers L{};
    int64_t need = 0;
    for (int l = 0; l < n_layers; ++l) {
        const int st = validate_lists(M, B, g, outs[l], in);
        if (st != AQLM_OK) return st;
        if (entries_bytes[l] < 0) return AQLM_ERR_SHAPE;
        if (outs[l] == 0 || batch == 0) continue;
        if (!tables[l] || !entries[l] || !codebooks[l] || !scales[l] || !ys[l]) return AQLM_ERR_NULL;
        if (!aligned(tables[l], 16) || !aligned(entries[l], 16) || !aligned(codebooks[l], 16) ||
            !aligned(ys[l], 16) || !aligned(scales[l], 2))
            return AQLM_ERR_ALIGN;
        const int i = L.n++;
        L.table[i] = static_cast<const uint32_t*>(tables[l]);
        L.entries[i] = static_cast<const uint32_t*>(entries[l]);
        L.cap[i] = (uint64_t)(entries_bytes[l] / 256);
        L.codebook[i] = codebooks[l];
        L.scales[i] = scales[l];
        L.y[i] = ys[l];
        L.out[i] = (int)outs[l];
        L.partial[i] = reinterpret_cast<float*>(need);   // offset for now
        need += lists_workspace_bytes_aligned(outs[l], in);
    }
    if (L.n == 0) return AQLM_OK;
    if (!x || !workspace) return AQLM_ERR_NULL;
    if (!aligned(x, 16) || !aligned(workspace, 16)) return AQLM_ERR_ALIGN;
    if (workspace_bytes < need) return AQLM_ERR_SHAPE;
    for (int i = 0; i < L.n; ++i)
        L.partial[i] = reinterpret_cast<float*>(static_cast<char*>(workspace) + reinterpret_cast<intptr_t>(L.partial[i]));
    return finish(launch_gemv_lists_fused(L, x, in, (hipStream_t)stream));
}

const char* aqlm_status_str(int status) {
    switch (status) {
        case AQLM_OK: return "AQLM_OK";
        case AQLM_ERR_NULL: return "AQLM_ERR_NULL: a required pointer is NULL (decode takes x == NULL)";
        case AQLM_ERR_SHAPE: return "AQLM_ERR_SHAPE: out/in/batch out of range or in % g != 0";
        case AQLM_ERR_SCHEME: return "AQLM_ERR_SCHEME: need 1 <= M <= 8, 1 <= B <= 16, g in {1,2,4,8,16,32}";
        case AQLM_ERR_ALIGN: return "AQLM_ERR_ALIGN: codes/codebooks/x/y need 16-byte, scales 2-byte alignment";
        case AQLM_ERR_HIP: return "AQLM_ERR_HIP: HIP runtime error at launch (see aqlm_last_hip_error)";
        case AQLM_ERR_SCRATCH:
            return "AQLM_ERR_SCRATCH: the problem needs more scratch than the allocation-free entry point's "
                   "static buffer holds (AQLM_LISTS_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown aqlm status";
    }
}

int aqlm_last_hip_error(void) { return g_last_hip_error; }

const char* aqlm_version(void) { return "0.1.0"; }

}  // extern "C"
