// pgq_gemm.hip -- the QAT forward's consumer GEMM with the weight dequantization fused in
// (gfx950, MFMA).
//
// STE fake quantization runs in the forward pass ("SubSixteen v2" card, PR #69, section Other):
// the layer's matmul consumes What[n][k] = bf16(fp32(code[n][k] * s_n)), the STE forward's
// dequantized weight.  Here the matmul reads the int8 codes and fp16 row scales instead of a
// materialised bf16 What, forms each bf16 weight in registers on its way into LDS, and runs
// the contraction on the matrix cores:
//
//     Y[m][n] = sum_k X[m][k] * What[n][k]      X bf16 [M x K], Y fp32 [M x N]
//
// Each product of two bf16 values is exact in fp32; the MFMA accumulates in fp32.
//
// Tiling: a workgroup of four wavefronts computes a 128 x 128 tile of Y; each wavefront a
// 64 x 64 quarter as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16.  Per 32-wide K step the
// workgroup stages X[128 x 32] and What[128 x 32] in LDS (rows padded to 40 halves), every
// thread loading 16 consecutive K elements of one row.  Operand layout of the instruction
// (checked on the device): lane l supplies row l % 32 of A (and column l % 32 of B) with
// k = 8 (l / 32) + i, i = 0..7; accumulator register j of lane l is row 8 (j / 4) +
// 4 (l / 32) + j % 4, column l % 32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pgq_desc.h"

namespace pgq {
namespace {

#define GLB __attribute__((address_space(1)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kPad = kBK + 8;            // LDS row pitch in halves (80 bytes)

__device__ __forceinline__ float half_to_float(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ uint16_t to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);     // round to nearest even
}

// flags: bit 0 = X rows are 16-byte loadable (ldx % 8 == 0, X 16-byte aligned),
//        bit 1 = code rows are 16-byte loadable (ldc % 16 == 0, codes 16-byte aligned)
__global__ void __launch_bounds__(256) pgq_qgemm_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       int64_t ldx, const int8_t* __restrict__ codes, int64_t ldc,
                                                       const uint16_t* __restrict__ scales, int64_t N,
                                                       float* __restrict__ y, int64_t ldy, uint32_t flags)
{
    __shared__ __align__(16) uint16_t As[kBM][kPad];
    __shared__ __align__(16) uint16_t Bs[kBN][kPad];
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // Workgroups are dealt to the 8 XCDs round-robin (workgroup i to XCD i mod 8) and each XCD has
    // its own L2, so consecutive tiles -- which share X rows -- are given to workgroups of the same
    // XCD: tile = (i mod 8)-th contiguous eighth of the tiles, element i / 8 of it (a bijection).
    const uint32_t gx = (uint32_t)((N + kBN - 1) / kBN);
    const uint32_t total = gridDim.x;
    const uint32_t wid = blockIdx.x;
    const uint32_t xcd = wid % 8u, per = total / 8u, rem = total % 8u;
    const uint32_t tile = (xcd < rem ? xcd * (per + 1u) : rem * (per + 1u) + (xcd - rem) * per) + wid / 8u;
    const int64_t m0 = (int64_t)(tile / gx) * kBM;
    const int64_t n0 = (int64_t)(tile % gx) * kBN;
    const int wm = (wave >> 1) * 64;
    const int wn = (wave & 1) * 64;
    // staging: thread t loads row t / 2, K elements 16 (t % 2) .. + 15 of the step
    const int lr = tid >> 1;
    const int lk = (tid & 1) * 16;
    const int64_t am = m0 + lr;
    const int64_t bn = n0 + lr;
    const float sb = bn < N ? half_to_float(scales[bn]) : 0.0f;
    const bool xvec = (flags & 1u) != 0;
    const bool cvec = (flags & 2u) != 0;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    for (int64_t k0 = 0; k0 < K; k0 += kBK) {
        const int64_t kb = k0 + lk;                      // first K index this thread stages
        uint16_t a[16];
        uint16_t b[16];
        if (am < M && xvec && kb + 16 <= K) {
            const GLB u32x4* p = (const GLB u32x4*)(x + am * ldx + kb);
            const u32x4 v0 = p[0], v1 = p[1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[2 * i] = (uint16_t)(v0[i] & 0xFFFFu);
                a[2 * i + 1] = (uint16_t)(v0[i] >> 16);
                a[8 + 2 * i] = (uint16_t)(v1[i] & 0xFFFFu);
                a[8 + 2 * i + 1] = (uint16_t)(v1[i] >> 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) a[i] = (am < M && kb + i < K) ? x[am * ldx + kb + i] : (uint16_t)0;
        }
        int8_t q[16];
        if (bn < N && cvec && kb + 16 <= K) {
            const u32x4 v = *(const GLB u32x4*)(codes + bn * ldc + kb);
#pragma unroll
            for (int i = 0; i < 16; ++i) q[i] = (int8_t)((v[i >> 2] >> (8 * (i & 3))) & 0xFFu);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) q[i] = (bn < N && kb + i < K) ? codes[bn * ldc + kb + i] : (int8_t)0;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) b[i] = to_bf16((float)q[i] * sb);   // the STE forward's weight

        __syncthreads();                                 // the previous step's fragments are read
        u32x4* as = reinterpret_cast<u32x4*>(&As[lr][lk]);
        u32x4* bs = reinterpret_cast<u32x4*>(&Bs[lr][lk]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            as[h] = u32x4{(uint32_t)a[8 * h] | ((uint32_t)a[8 * h + 1] << 16), (uint32_t)a[8 * h + 2] | ((uint32_t)a[8 * h + 3] << 16),
                          (uint32_t)a[8 * h + 4] | ((uint32_t)a[8 * h + 5] << 16), (uint32_t)a[8 * h + 6] | ((uint32_t)a[8 * h + 7] << 16)};
            bs[h] = u32x4{(uint32_t)b[8 * h] | ((uint32_t)b[8 * h + 1] << 16), (uint32_t)b[8 * h + 2] | ((uint32_t)b[8 * h + 3] << 16),
                          (uint32_t)b[8 * h + 4] | ((uint32_t)b[8 * h + 5] << 16), (uint32_t)b[8 * h + 6] | ((uint32_t)b[8 * h + 7] << 16)};
        }
        __syncthreads();

#pragma unroll
        for (int kk = 0; kk < kBK; kk += 16) {
            const int ko = kk + 8 * (lane >> 5);
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fa[i] = *reinterpret_cast<const bf16x8*>(&As[wm + 32 * i + (lane & 31)][ko]);
                fb[i] = *reinterpret_cast<const bf16x8*>(&Bs[wn + 32 * i + (lane & 31)][ko]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < M && col < N) y[row * ldy + col] = acc[i][j][r];
            }
        }
}

}  // namespace

int launch_qgemm(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* codes, int64_t ldc,
                 const uint16_t* scales, int64_t N, float* y, int64_t ldy, uint32_t flags, void* stream)
{
    const uint64_t tiles = (uint64_t)((N + kBN - 1) / kBN) * (uint64_t)((M + kBM - 1) / kBM);
    if (tiles > 0xFFFFFFFFull) return (int)hipErrorInvalidValue;
    const dim3 grid((unsigned)tiles);
    void* args[] = {&x, &M, &K, &ldx, &codes, &ldc, &scales, &N, &y, &ldy, &flags};
    return (int)launch_plain(reinterpret_cast<const void*>(&pgq_qgemm_kernel), grid, dim3(256), args, stream);
}

}  // namespace pgq
