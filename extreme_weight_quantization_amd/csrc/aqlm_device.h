// Device-side helpers shared by the AQLM kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aqlm {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Scheme ids used as template parameters.
// kSchemeGeneric: any other (M, B, g), served by the kernels of generic.hip.
// kSchemeB8M1/M4/M8: the other 2-bit schemes with B = 8 (1x8 g4, 4x8 g16,
// 8x8 g32; 2x8 g8 is kScheme2x8), whose GEMV runs the 2x8 product's kernel.
enum Scheme : int { kScheme2x8 = 0, kScheme1x16 = 1, kSchemeGeneric = 2, kSchemeB8M1 = 3, kSchemeB8M4 = 4,
                    kSchemeB8M8 = 5 };

// Codebooks of a 2-bit B = 8 scheme (g = 4 M), 0 for the others.
constexpr int b8_codebooks(int scheme) {
    return scheme == kScheme2x8 ? 2 : scheme == kSchemeB8M1 ? 1 : scheme == kSchemeB8M4 ? 4
         : scheme == kSchemeB8M8 ? 8 : 0;
}

constexpr int kGroup = 8;          // g: inputs per group
constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kCodewords2x8 = 256; // 2^B for B = 8

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(f16x8 v) { return __builtin_bit_cast(u32x4, v); }

// 16x16x32 fp16 matrix-core product with fp32 accumulation:
//   D[i][j] = C[i][j] + sum_k A[i][k] * B[k][j],
// lane l supplies A[l % 16][8*(l/16) .. +8) and B[8*(l/16) .. +8)[l % 16] and
// holds D[4*(l/16) + r][l % 16] for r = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Streaming (non-temporal) 16-byte load: codes are read exactly once.
__device__ __forceinline__ u32x4 load_nt16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// A generic pointer into the workgroup's LDS as the LDS address space, for the
// direct-to-LDS loads (__builtin_amdgcn_global_load_lds).
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(void* p) {
    return (__attribute__((address_space(3))) void*)p;
}

// s_waitcnt immediates for __builtin_amdgcn_s_waitcnt, which, unlike a wait in
// inline assembly, the compiler's own wait placement sees.  vmcnt sits in bits
// 0-3 and 14-15, expcnt in 4-6, lgkmcnt in 8-11.
// vmcnt(n) lgkmcnt(0), the export counter at its maximum (n < 16):
constexpr int wait_vm_lgkm0(int n) { return n | (7 << 4); }
// lgkmcnt(0), the vector-memory and export counters at their maxima:
constexpr int kWaitLgkm0 = 0xF | (3 << 14) | (7 << 4);

}  // namespace aqlm
