// Host-only driver of the C ABI's argument validation, built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host pass (tests/test_host_sanitizers.py).
//
// Every launcher that the entry points call is replaced by a stub that only counts
// the call (and can report a HIP error), so nothing here touches a GPU: the
// "device" pointers are host buffers that no stub dereferences.  The driver then
// calls every entry point with valid arguments, NULL pointers, misaligned
// pointers, out-of-range and extreme sizes (INT64_MIN/MAX), and host arrays of
// exactly n_layers entries, and checks each status and launch count.  The
// sanitizers report any out-of-bounds host read, signed overflow or other
// undefined behaviour in the validation itself.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/aqlm.h"
#include "../../extreme_weight_quantization_amd/csrc/aqlm_launch.h"

namespace {
int g_launches = 0;
hipError_t g_result = hipSuccess;
int g_failures = 0;

hipError_t stub() {
    ++g_launches;
    return g_result;
}
}  // namespace

namespace aqlm {
hipError_t launch_decode_generic(const GenericScheme&, const void*, const void*, const void*, void*, int64_t,
                                 int64_t, hipStream_t) { return stub(); }
hipError_t launch_gemv_generic(const GenericScheme&, const void*, const void*, const void*, const void*, void*,
                               int64_t, int64_t, int64_t, hipStream_t) { return stub(); }
hipError_t launch_encode_greedy(const void*, const void*, const void*, void*, int, int, int, int64_t, int64_t,
                                hipStream_t) { return stub(); }
hipError_t launch_kmeans_init(const void*, const void*, const int64_t*, void*, void*, void*, int, int, int, int64_t,
                              int64_t, int, hipStream_t) { return stub(); }
int64_t kmeans_workspace_bytes(int, int B, int g) { return ((int64_t)1 << B) * (g * 12 + 8) + 16; }
hipError_t launch_gemm_generic(const GenericScheme&, const void*, const void*, const void*, const void*, void*,
                               int64_t, int64_t, int64_t, hipStream_t) { return stub(); }
hipError_t launch_decode(int, const void*, const void*, const void*, void*, int64_t, int64_t, hipStream_t) {
    return stub();
}
hipError_t launch_gemv_fused(int, GemvLayers, const void*, int64_t, int64_t, hipStream_t) { return stub(); }
hipError_t launch_gemv(int, const void*, const void*, const void*, const void*, void*, int64_t, int64_t, int64_t,
                       hipStream_t) { return stub(); }
hipError_t launch_gemm_pipe_2x8(const void*, const void*, const void*, const void*, void*, int64_t, int64_t,
                                int64_t, hipStream_t) { return stub(); }
hipError_t launch_gemm_pipe_1x8g4(const void*, const void*, const void*, const void*, void*, int64_t, int64_t,
                                  int64_t, hipStream_t) { return stub(); }
hipError_t launch_gemm_pipe_4x8g16(const void*, const void*, const void*, const void*, void*, int64_t, int64_t,
                                  int64_t, hipStream_t) { return stub(); }
hipError_t launch_gemm_dense(const void*, const void*, void*, int64_t, int64_t, int64_t, hipStream_t) {
    return stub();
}
hipError_t launch_gemm(int, const void*, const void*, const void*, const void*, void*, int64_t, int64_t, int64_t,
                       hipStream_t) { return stub(); }
int64_t lists_workspace_bytes_aligned(int64_t out, int64_t) { return (out * 32 + 255) / 256 * 256; }
hipError_t launch_gemv_lists_fused(ListsLayers, const void*, int64_t, hipStream_t) { return stub(); }
int64_t lists_table_bytes(int64_t out, int64_t) { return out * 8 + 8; }
int64_t lists_workspace_bytes(int64_t out, int64_t) { return out * 32; }
hipError_t launch_lists_plan(const void*, int64_t, int64_t, void*, hipStream_t) { return stub(); }
hipError_t launch_lists_fill(const void*, int64_t, int64_t, const void*, void*, int64_t, hipStream_t) {
    return stub();
}
hipError_t launch_gemv_lists(const void*, const void*, int64_t, const void*, const void*, const void*, void*,
                             void*, int64_t, int64_t, hipStream_t) { return stub(); }
uint64_t packed_code_words(int M, int B, int g, int64_t out, int64_t in) {
    return ((uint64_t)out * (uint64_t)(in / g) * (uint64_t)M * (uint64_t)B + 31) / 32;
}
hipError_t launch_pack_codes(const void*, void*, int, int, int, int64_t, int64_t, hipStream_t) { return stub(); }
hipError_t lists_scratch(void** ptr) {
    static float fake[16];
    *ptr = fake;
    return hipSuccess;
}
}  // namespace aqlm

#define CHECK(expr, want_status, want_launches)                                                        \
    do {                                                                                               \
        const int before_ = g_launches;                                                                \
        const int got_ = (expr);                                                                       \
        if (got_ != (want_status) || g_launches - before_ != (want_launches)) {                        \
            fprintf(stderr, "line %d: %s -> status %d (want %d), launches %d (want %d)\n", __LINE__,   \
                    #expr, got_, (int)(want_status), g_launches - before_, (int)(want_launches));      \
            ++g_failures;                                                                              \
        }                                                                                              \
    } while (0)

int main() {
    const int64_t I64_MAX = INT64_MAX, I64_MIN = INT64_MIN;
    // 16-byte aligned host buffers standing in for device memory (never dereferenced)
    char* buf = static_cast<char*>(aligned_alloc(256, 1 << 16));
    void *c = buf, *cb = buf + 256, *s = buf + 512, *x = buf + 768, *y = buf + 1024, *ws = buf + 1280;
    void* odd = buf + 8;   // 8-byte aligned, not 16
    void* st = nullptr;

    // ---- aqlm_linear_gemv / gemm / decode
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 8, 64, 256, 1, st), AQLM_OK, 1);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 1, 16, 8, 64, 256, 16, st), AQLM_OK, 1);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 3, 5, 8, 64, 256, 3, st), AQLM_OK, 1);
    CHECK(aqlm_linear_gemv(nullptr, cb, s, x, y, 2, 8, 8, 64, 256, 1, st), AQLM_ERR_NULL, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, nullptr, y, 2, 8, 8, 64, 256, 1, st), AQLM_ERR_NULL, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, odd, 2, 8, 8, 64, 256, 1, st), AQLM_ERR_ALIGN, 0);
    CHECK(aqlm_linear_gemv(c, cb, buf + 1, x, y, 2, 8, 8, 64, 256, 1, st), AQLM_ERR_ALIGN, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 5, 64, 256, 1, st), AQLM_ERR_SCHEME, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 9, 8, 8, 64, 256, 1, st), AQLM_ERR_SCHEME, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 1, 17, 8, 64, 256, 1, st), AQLM_ERR_SCHEME, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 8, 64, 252, 1, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 8, 64, 256, 17, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 8, 64, 256, -1, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 8, I64_MAX, 256, 1, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 8, I64_MIN, 256, 1, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 8, 64, I64_MAX, 1, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 8, 64, I64_MIN, 1, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 8, 64, 256, I64_MIN, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv(nullptr, nullptr, nullptr, nullptr, nullptr, 2, 8, 8, 0, 256, 1, st), AQLM_OK, 0);
    CHECK(aqlm_linear_gemv(nullptr, nullptr, nullptr, nullptr, nullptr, 2, 8, 8, 64, 256, 0, st), AQLM_OK, 0);
    CHECK(aqlm_linear_gemm(c, cb, s, x, y, 2, 8, 8, 64, 256, 2048, st), AQLM_OK, 1);
    CHECK(aqlm_linear_gemm(c, cb, s, x, y, 1, 8, 4, 64, 256, 2048, st), AQLM_OK, 1);
    CHECK(aqlm_linear_gemm(c, cb, s, x, y, 2, 8, 8, 64, 256, I64_MAX, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemm(c, cb, s, x, y, 2, 8, 8, (int64_t)INT32_MAX - 16, 256, (int64_t)INT32_MAX - 256, st),
          AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_decode(c, cb, s, nullptr, y, 2, 8, 8, 64, 256, 0, st), AQLM_OK, 1);
    CHECK(aqlm_linear_decode(c, cb, s, x, y, 2, 8, 8, 64, 256, 0, st), AQLM_ERR_NULL, 0);
    CHECK(aqlm_linear_decode(c, cb, s, nullptr, y, 2, 8, 8, (int64_t)1 << 30, 1 << 20, 0, st), AQLM_ERR_SHAPE, 0);

    // ---- the HIP error path: the stub's error comes back as AQLM_ERR_HIP and is kept per thread
    g_result = hipErrorInvalidValue;
    CHECK(aqlm_linear_gemv(c, cb, s, x, y, 2, 8, 8, 64, 256, 1, st), AQLM_ERR_HIP, 1);
    if (aqlm_last_hip_error() != (int)hipErrorInvalidValue) {
        fprintf(stderr, "aqlm_last_hip_error %d\n", aqlm_last_hip_error());
        ++g_failures;
    }
    g_result = hipSuccess;

    // ---- fused GEMV: host arrays of exactly n entries (over-reads show up under ASan)
    for (int n = 1; n <= AQLM_FUSED_MAX_LAYERS; ++n) {
        const void** cs = static_cast<const void**>(malloc(n * sizeof(void*)));
        const void** cbs = static_cast<const void**>(malloc(n * sizeof(void*)));
        const void** ss = static_cast<const void**>(malloc(n * sizeof(void*)));
        void** ys = static_cast<void**>(malloc(n * sizeof(void*)));
        int64_t* outs = static_cast<int64_t*>(malloc(n * sizeof(int64_t)));
        for (int l = 0; l < n; ++l) {
            cs[l] = c; cbs[l] = cb; ss[l] = s; ys[l] = y; outs[l] = 64 * (l + 1);
        }
        CHECK(aqlm_linear_gemv_fused(n, cs, cbs, ss, outs, x, ys, 2, 8, 8, 256, 4, st), AQLM_OK, 1);
        CHECK(aqlm_linear_gemv_fused(n, cs, cbs, ss, outs, x, ys, 3, 5, 8, 256, 4, st), AQLM_OK, n);
        outs[n - 1] = 0;   // an empty layer is skipped
        CHECK(aqlm_linear_gemv_fused(n, cs, cbs, ss, outs, x, ys, 2, 8, 8, 256, 4, st), AQLM_OK, n > 1 ? 1 : 0);
        outs[n - 1] = I64_MIN;
        CHECK(aqlm_linear_gemv_fused(n, cs, cbs, ss, outs, x, ys, 2, 8, 8, 256, 4, st), AQLM_ERR_SHAPE, 0);
        outs[n - 1] = 64;
        ys[n - 1] = odd;
        CHECK(aqlm_linear_gemv_fused(n, cs, cbs, ss, outs, x, ys, 2, 8, 8, 256, 4, st), AQLM_ERR_ALIGN, 0);
        free(cs); free(cbs); free(ss); free(ys); free(outs);
    }
    {
        const void* one[1] = {c};
        void* yo[1] = {y};
        int64_t o1[1] = {64};
        CHECK(aqlm_linear_gemv_fused(0, one, one, one, o1, x, yo, 2, 8, 8, 256, 1, st), AQLM_ERR_SHAPE, 0);
        CHECK(aqlm_linear_gemv_fused(9, one, one, one, o1, x, yo, 2, 8, 8, 256, 1, st), AQLM_ERR_SHAPE, 0);
        CHECK(aqlm_linear_gemv_fused(1, nullptr, one, one, o1, x, yo, 2, 8, 8, 256, 1, st), AQLM_ERR_NULL, 0);
        CHECK(aqlm_linear_gemv_fused(1, one, one, one, nullptr, x, yo, 2, 8, 8, 256, 1, st), AQLM_ERR_NULL, 0);
    }

    // ---- bit-packed codes: 4-byte aligned streams
    int64_t pb = 0;
    CHECK(aqlm_packed_codes_bytes(1, 12, 4, 64, 512, &pb), AQLM_OK, 0);
    if (pb != 64 * 128 * 12 / 8) { fprintf(stderr, "packed bytes %lld\n", (long long)pb); ++g_failures; }
    CHECK(aqlm_packed_codes_bytes(1, 12, 4, I64_MAX, 512, &pb), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_packed_codes_bytes(1, 17, 4, 64, 512, &pb), AQLM_ERR_SCHEME, 0);
    CHECK(aqlm_pack_codes(c, y, 1, 12, 4, 64, 512, st), AQLM_OK, 1);
    CHECK(aqlm_pack_codes(c, buf + 2, 1, 12, 4, 64, 512, st), AQLM_ERR_ALIGN, 0);
    CHECK(aqlm_pack_codes(nullptr, y, 1, 12, 4, 64, 512, st), AQLM_ERR_NULL, 0);
    CHECK(aqlm_linear_gemv_packed(buf + 4, cb, s, x, y, 3, 5, 8, 64, 512, 4, st), AQLM_OK, 1);
    CHECK(aqlm_linear_gemv_packed(buf + 2, cb, s, x, y, 3, 5, 8, 64, 512, 4, st), AQLM_ERR_ALIGN, 0);
    CHECK(aqlm_linear_gemm_packed(buf + 4, cb, s, x, y, 2, 12, 8, 64, 512, 300, st), AQLM_OK, 1);
    CHECK(aqlm_linear_decode_packed(buf + 4, cb, s, nullptr, y, 2, 12, 8, 64, 512, 0, st), AQLM_OK, 1);
    CHECK(aqlm_linear_decode_packed(buf + 4, cb, s, x, y, 2, 12, 8, 64, 512, 0, st), AQLM_ERR_NULL, 0);
    CHECK(aqlm_linear_gemv_packed(buf + 4, cb, s, x, y, 3, 5, 8, I64_MIN, 512, 4, st), AQLM_ERR_SHAPE, 0);

    // ---- two-pass prefill
    int64_t nb = -1;
    CHECK(aqlm_gemm_dequant_workspace_bytes(2, 8, 8, 64, 256, &nb), AQLM_OK, 0);
    if (nb != 64 * 256 * 2) { fprintf(stderr, "dequant workspace %lld\n", (long long)nb); ++g_failures; }
    CHECK(aqlm_gemm_dequant_workspace_bytes(2, 8, 8, I64_MAX, 256, &nb), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_gemm_dequant_workspace_bytes(2, 8, 8, 64, 256, nullptr), AQLM_ERR_NULL, 0);
    CHECK(aqlm_linear_gemm_dequant(c, cb, s, x, y, ws, 64 * 256 * 2, 2, 8, 8, 64, 256, 16, st), AQLM_OK, 2);
    CHECK(aqlm_linear_gemm_dequant(c, cb, s, x, y, ws, 64 * 256 * 2 - 1, 2, 8, 8, 64, 256, 16, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemm_dequant(c, cb, s, x, y, nullptr, 1 << 20, 2, 8, 8, 64, 256, 16, st), AQLM_ERR_NULL, 0);
    CHECK(aqlm_linear_gemm_dequant(c, cb, s, x, y, odd, 1 << 20, 2, 8, 8, 64, 256, 16, st), AQLM_ERR_ALIGN, 0);
    CHECK(aqlm_linear_gemm_dequant(c, cb, s, x, y, nullptr, 0, 2, 8, 8, 64, 200, 16, st), AQLM_OK, 1);
    CHECK(aqlm_linear_gemm_dequant(c, cb, s, x, y, ws, I64_MIN, 2, 8, 8, 64, 256, 16, st), AQLM_ERR_SHAPE, 0);

    // ---- encoder and k-means
    CHECK(aqlm_encode_greedy(x, s, cb, c, 2, 8, 8, 64, 256, st), AQLM_OK, 1);
    CHECK(aqlm_encode_greedy(x, s, cb, c, 2, 8, 8, I64_MIN, 256, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_encode_greedy(x, s, cb, nullptr, 2, 8, 8, 64, 256, st), AQLM_ERR_NULL, 0);
    int64_t kb = 0;
    CHECK(aqlm_kmeans_workspace_bytes(2, 8, 8, &kb), AQLM_OK, 0);
    const int64_t* seeds = static_cast<const int64_t*>(ws);
    CHECK(aqlm_kmeans_init(x, s, seeds, cb, c, ws, kb, 2, 8, 8, 64, 256, 3, st), AQLM_OK, 1);
    CHECK(aqlm_kmeans_init(x, s, seeds, cb, c, ws, kb - 1, 2, 8, 8, 64, 256, 3, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_kmeans_init(x, s, seeds, cb, c, ws, kb, 2, 8, 8, 64, 256, -1, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_kmeans_init(x, s, seeds, cb, c, ws, kb, 2, 8, 8, 64, 256, AQLM_KMEANS_MAX_ITERS + 1, st),
          AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_kmeans_init(x, s, nullptr, cb, c, ws, kb, 2, 8, 8, 64, 256, 3, st), AQLM_ERR_NULL, 0);
    CHECK(aqlm_kmeans_init(x, s, reinterpret_cast<const int64_t*>(buf + 4), cb, c, ws, kb, 2, 8, 8, 64, 256, 3, st),
          AQLM_ERR_ALIGN, 0);

    // ---- slice lists
    int64_t tb = 0, wb = 0;
    CHECK(aqlm_lists_table_bytes(1, 16, 8, 4096, 4096, &tb), AQLM_OK, 0);
    CHECK(aqlm_lists_workspace_bytes(1, 16, 8, 4096, 4096, &wb), AQLM_OK, 0);
    CHECK(aqlm_lists_table_bytes(2, 8, 8, 4096, 4096, &tb), AQLM_ERR_SCHEME, 0);
    CHECK(aqlm_lists_table_bytes(1, 16, 8, I64_MAX, 4096, &tb), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_lists_table_bytes(1, 16, 8, (int64_t)1 << 30, 1 << 20, &tb), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_lists_plan(c, ws, 1, 16, 8, 64, 256, st), AQLM_OK, 1);
    CHECK(aqlm_lists_plan(nullptr, ws, 1, 16, 8, 0, 256, st), AQLM_OK, 1);
    CHECK(aqlm_lists_plan(nullptr, ws, 1, 16, 8, 64, 256, st), AQLM_ERR_NULL, 0);
    CHECK(aqlm_lists_fill(c, ws, y, 4096, 1, 16, 8, 64, 256, st), AQLM_OK, 1);
    CHECK(aqlm_lists_fill(c, ws, y, -1, 1, 16, 8, 64, 256, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv_lists(ws, y, 4096, cb, s, x, y, ws, 64 * 32, 1, 16, 8, 64, 256, 1, st), AQLM_OK, 1);
    CHECK(aqlm_linear_gemv_lists(ws, y, 4096, cb, s, x, y, ws, 64 * 32 - 1, 1, 16, 8, 64, 256, 1, st),
          AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv_lists(ws, y, 4096, cb, s, x, y, ws, 64 * 32, 1, 16, 8, 64, 256, 2, st), AQLM_ERR_SHAPE, 0);
    CHECK(aqlm_linear_gemv_lists(ws, y, I64_MIN, cb, s, x, y, ws, 64 * 32, 1, 16, 8, 64, 256, 1, st),
          AQLM_ERR_SHAPE, 0);
    // allocation-free variant: the stub's lists_workspace_bytes is out * 32, so 131072 rows fill 4 MiB
    CHECK(aqlm_linear_gemv_lists_noalloc(ws, y, 4096, cb, s, x, y, 1, 16, 8, 64, 256, 1, st), AQLM_OK, 1);
    CHECK(aqlm_linear_gemv_lists_noalloc(ws, y, 4096, cb, s, x, y, 1, 16, 8, 131072, 256, 1, st), AQLM_OK, 1);
    CHECK(aqlm_linear_gemv_lists_noalloc(ws, y, 4096, cb, s, x, y, 1, 16, 8, 131073, 256, 1, st),
          AQLM_ERR_SCRATCH, 0);
    CHECK(aqlm_linear_gemv_lists_noalloc(ws, y, 4096, cb, s, x, nullptr, 1, 16, 8, 64, 256, 1, st), AQLM_ERR_NULL, 0);
    CHECK(aqlm_linear_gemv_lists_noalloc(ws, y, 4096, cb, s, x, odd, 1, 16, 8, 64, 256, 1, st), AQLM_ERR_ALIGN, 0);
    CHECK(aqlm_linear_gemv_lists_noalloc(ws, y, 4096, cb, s, x, y, 2, 8, 8, 64, 256, 1, st), AQLM_ERR_SCHEME, 0);
    CHECK(aqlm_linear_gemv_lists_noalloc(nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, 1, 16, 8, 0, 256,
                                         1, st), AQLM_OK, 0);
    CHECK(aqlm_linear_gemv_lists_noalloc(ws, y, I64_MIN, cb, s, x, y, 1, 16, 8, 64, 256, 1, st), AQLM_ERR_SHAPE, 0);
    for (int n = 1; n <= AQLM_FUSED_MAX_LAYERS; ++n) {
        const void** t = static_cast<const void**>(malloc(n * sizeof(void*)));
        const void** e = static_cast<const void**>(malloc(n * sizeof(void*)));
        const void** cbs = static_cast<const void**>(malloc(n * sizeof(void*)));
        const void** ss = static_cast<const void**>(malloc(n * sizeof(void*)));
        void** ys = static_cast<void**>(malloc(n * sizeof(void*)));
        int64_t* eb = static_cast<int64_t*>(malloc(n * sizeof(int64_t)));
        int64_t* outs = static_cast<int64_t*>(malloc(n * sizeof(int64_t)));
        for (int l = 0; l < n; ++l) {
            t[l] = ws; e[l] = y; cbs[l] = cb; ss[l] = s; ys[l] = y; eb[l] = 4096; outs[l] = 64 + l;
        }
        int64_t fb = 0;
        CHECK(aqlm_lists_fused_workspace_bytes(n, outs, 1, 16, 8, 256, &fb), AQLM_OK, 0);
        CHECK(aqlm_linear_gemv_lists_fused(n, t, e, eb, cbs, ss, outs, x, ys, ws, fb, 1, 16, 8, 256, 1, st),
              AQLM_OK, 1);
        CHECK(aqlm_linear_gemv_lists_fused(n, t, e, eb, cbs, ss, outs, x, ys, ws, fb - 1, 1, 16, 8, 256, 1, st),
              AQLM_ERR_SHAPE, 0);
        eb[n - 1] = -1;
        CHECK(aqlm_linear_gemv_lists_fused(n, t, e, eb, cbs, ss, outs, x, ys, ws, fb, 1, 16, 8, 256, 1, st),
              AQLM_ERR_SHAPE, 0);
        free(t); free(e); free(cbs); free(ss); free(ys); free(eb); free(outs);
    }

#ifdef AQLM_PLANT_OVERREAD
    {   // a deliberate host-array over-read: proves the sanitizer build is armed
        const void** one = static_cast<const void**>(malloc(sizeof(void*)));
        void** yo = static_cast<void**>(malloc(sizeof(void*)));
        int64_t* o1 = static_cast<int64_t*>(malloc(sizeof(int64_t)));
        one[0] = c; yo[0] = y; o1[0] = 64;
        aqlm_linear_gemv_fused(2, one, one, one, o1, x, yo, 2, 8, 8, 256, 1, st);
        free(one); free(yo); free(o1);
    }
#endif

    // ---- helpers
    for (int code = -3; code < 10; ++code)
        if (aqlm_status_str(code) == nullptr || strlen(aqlm_status_str(code)) == 0) ++g_failures;
    if (aqlm_version() == nullptr) ++g_failures;

    free(buf);
    if (g_failures) {
        fprintf(stderr, "%d validation checks failed\n", g_failures);
        return 1;
    }
    printf("api validation ok\n");
    return 0;
}
