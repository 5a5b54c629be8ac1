// pgq_gemm.hip -- the QAT forward's consumer GEMM with the weight dequantization fused in
// (gfx950, MFMA).
//
// STE fake quantization runs in the forward pass ("SubSixteen v2" card, PR #69, section Other):
// the layer's matmul consumes What[n][k] = bf16(fp32(code[n][k] * s_n)), the STE forward's
// dequantized weight.  Here the matmul reads the int8 codes and fp16 row scales instead of a
// materialised bf16 What, forms each bf16 weight in registers, and runs the contraction on the
// matrix cores:
//
//     Y[m][n] = sum_k X[m][k] * What[n][k]      X bf16 [M x K], Y fp32 [M x N]
//
// Each product of two bf16 values is exact in fp32; the MFMA accumulates in fp32.
//
// Two kernels.  The main one (pgq_qgemm_kernel) takes 16-byte loadable rows and K a multiple of
// 16: a workgroup of four wavefronts computes a 256 x 128 tile of Y, each wavefront a 128 x 64
// part as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16.  X[256 x 64] and the raw int8 codes[128 x 64]
// of each 64-wide K step go from global memory straight into LDS (buffer loads with the LDS
// destination, no registers on the way), double-buffered, so the next step's loads are in
// flight while the matrix cores work on this one; a lane past M, N or K gets zeros from the
// buffer range check.  Each wavefront turns its own code fragments into bf16(code * s_n) in
// registers.  Y leaves through an LDS transpose as 16-byte non-temporal stores.  The generic
// kernel (pgq_qgemm_generic_kernel) takes any shape: element loads through registers into LDS.
//
// Operand layout of the instruction (checked on the device): lane l supplies row l % 32 of A
// (and column l % 32 of B) with 8 consecutive k, the lanes 32..63 the next 8; accumulator
// register j of lane l is row 8 (j / 4) + 4 (l / 32) + j % 4, column l % 32.  Which of the
// tile's k a lane half supplies in which instruction is free as long as A and B agree: in the
// main kernel, lane half h supplies k = 16 h + 8 t .. + 7 of a 32-wide block in the block's
// t-th instruction, so that a lane reads its 16 contiguous k of each row with one LDS read.
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

// Y element: fp32, or bf16 (round to nearest even of the fp32 result) as it leaves
template <typename YT>
__device__ __forceinline__ YT y_of(float v);
template <>
__device__ __forceinline__ float y_of<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t y_of<uint16_t>(float v) { return to_bf16(v); }

// flags: bit 0 = X rows are 16-byte loadable (ldx % 8 == 0, X 16-byte aligned),
//        bit 1 = code rows are 16-byte loadable (ldc % 16 == 0, codes 16-byte aligned)
template <typename YT>
__global__ void __launch_bounds__(256) pgq_qgemm_generic_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       int64_t ldx, const int8_t* __restrict__ codes, int64_t ldc,
                                                       const uint16_t* __restrict__ scales, int64_t N,
                                                       YT* __restrict__ y, int64_t ldy, uint32_t flags)
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
    const float sb = (K > 0 && bn < N) ? half_to_float(scales[bn]) : 0.0f;   // K = 0: nothing is read
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
                if (row < M && col < N) y[row * ldy + col] = y_of<YT>(acc[i][j][r]);
            }
        }
}


// ---- main kernel: direct-to-LDS loads, double-buffered ---------------------------------------------
constexpr int kTK = 64;                        // K per stage
constexpr int kIB = 4;                         // 32-row MFMA blocks per wavefront
constexpr int kTM = 64 * kIB;                  // workgroup rows (2 wavefronts along M): 256
constexpr int kTN = 128;                       // workgroup columns (2 wavefronts along N)
constexpr int kXI = kTM / 32;                  // X load instructions per thread per stage
constexpr int kAS = kTM * kTK * 2;             // X bytes per stage (256 rows x 128 B)
constexpr int kBS = kTN * kTK;                 // code bytes per stage (128 rows x 64 B)
constexpr uint32_t kOOB = 0x80000000u;         // a buffer offset past every range: the load returns 0

// LDS slots are 16-byte granules.  X rows hold 8 granules, code rows 4; granule g of row r is
// stored in slot g ^ swz(r) of the row, so that the 32 rows a fragment read touches (same
// granule) spread over distinct banks in every group of 8 and of 16 lanes.
__device__ __forceinline__ int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_b(int r) { return (((r >> 1) & 1) ^ ((r >> 3) & 1)) | (((r >> 2) & 1) << 1); }

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// every wave's LDS reads are complete, then the workgroup barrier (the asm keeps the compiler
// from moving memory operations across it)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t pk_bf16(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));   // round to nearest even
}

// 16 int8 codes (one 16-byte LDS granule) -> two bf16x8 fragments of bf16(code * s): with
// u = byte + 128 from the biased byte, fma(u, s, -128 s) = code * s exactly (at most 7 + 11
// significant bits), then round to bf16
__device__ __forceinline__ void codes_to_bf16(u32x4 q, float s, float s128, bf16x8& lo, bf16x8& hi)
{
    float v[16];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t b = q[w] ^ 0x80808080u;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * w + e] = __builtin_fmaf((float)((b >> (8 * e)) & 0xFFu), s, s128);
    }
    u32x4 a, c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = pk_bf16(v[2 * e], v[2 * e + 1]);
        c[e] = pk_bf16(v[8 + 2 * e], v[8 + 2 * e + 1]);
    }
    lo = __builtin_bit_cast(bf16x8, a);
    hi = __builtin_bit_cast(bf16x8, c);
}

// A workgroup of four wavefronts computes a 256 x 128 tile of Y; wavefront w a 128 x 64 part
// (rows 128 (w / 2), columns 64 (w % 2)) as 4 x 2 blocks of 32 x 32.  Occupancy floor of two
// wavefronts per SIMD (the register budget the 128 accumulators leave), matching the two
// workgroups per compute unit that the 80 KB of LDS allow.
template <typename YT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
pgq_qgemm_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, const int8_t* __restrict__ codes,
                 int64_t ldc, const uint16_t* __restrict__ scales, int64_t N, YT* __restrict__ y, int64_t ldy,
                 int32_t yvec)
{
    __shared__ __align__(16) uint8_t lds[2 * (kAS + kBS)];
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // tiles sharing X rows go to workgroups of one XCD (workgroup i runs on XCD i mod 8)
    const uint32_t gx = (uint32_t)((N + kTN - 1) / kTN);
    const uint32_t total = gridDim.x;
    const uint32_t wid = blockIdx.x;
    const uint32_t xcd = wid % 8u, per = total / 8u, rem = total % 8u;
    const uint32_t tile = (xcd < rem ? xcd * (per + 1u) : rem * (per + 1u) + (xcd - rem) * per) + wid / 8u;
    const int64_t m0 = (int64_t)(tile / gx) * kTM;
    const int64_t n0 = (int64_t)(tile % gx) * kTN;
    const int mrows = (int)min((int64_t)kTM, M - m0);
    const int nrows = (int)min((int64_t)kTN, N - n0);
    // buffer ranges over this tile's rows (the host keeps them below 2^31 bytes)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + m0 * ldx), 0, (int)((int64_t)mrows * ldx * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(codes + n0 * ldc), 0, (int)((int64_t)nrows * ldc), 0x00020000);

    // load slots: X instruction c covers slot p = 256 c + tid, row 32 c + tid / 8, granule
    // (tid % 8) ^ swz_a(row), which is the same for every c; codes instruction c: row 64 c + tid / 4,
    // granule (tid % 4) ^ swz_b(row), also the same for every c.  Each instruction of a wave
    // fills 1 KB of consecutive LDS.
    const int xr0 = tid >> 3;
    const int xg = (tid & 7) ^ swz_a(xr0);
    const int cr0 = tid >> 2;
    const int cg = (tid & 3) ^ swz_b(cr0);
    const uint32_t xo0 = (uint32_t)(xr0 * ldx + 8 * xg) * 2u;
    const uint32_t co0 = (uint32_t)(cr0 * ldc + 16 * cg);
    const uint32_t xstep = (uint32_t)(64 * ldx);       // 32 rows of X, bytes
    const uint32_t cstep = (uint32_t)(64 * ldc);       // 64 rows of codes, bytes
    const int nst = (int)((K + kTK - 1) / kTK);
    auto issue = [&](int st) {
        const int k0 = st * kTK;
        uint8_t* la = lds + (st & 1) * (kAS + kBS);
        uint8_t* lb = la + kAS;
        const bool xk_ok = k0 + 8 * xg < K;
        const bool ck_ok = k0 + 16 * cg < K;
        // a lane past M, N or K reads offset kOOB (mask arithmetic, so that the compiler keeps one
        // load per slot rather than branching around two)
#pragma unroll
        for (int c = 0; c < kXI; ++c) {
            const uint32_t bad = 0u - (uint32_t)!(xk_ok && xr0 + 32 * c < mrows);
            const uint32_t o = ((xo0 + (uint32_t)c * xstep + (uint32_t)k0 * 2u) & ~bad) | (kOOB & bad);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr)(la + (c * 256 + wave * 64) * 16), 16, o, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint32_t bad = 0u - (uint32_t)!(ck_ok && cr0 + 64 * c < nrows);
            const uint32_t o = ((co0 + (uint32_t)c * cstep + (uint32_t)k0) & ~bad) | (kOOB & bad);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, (lds_ptr)(lb + (c * 256 + wave * 64) * 16), 16, o, 0, 0, 0);
        }
    };

    const int wm = (wave >> 1) * (32 * kIB);
    const int wn = (wave & 1) * 64;
    const int r32 = lane & 31;
    const int h = lane >> 5;
    // the scales of this lane's two weight rows (columns of Y)
    float sc[2], sc128[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wn + 32 * j + r32;
        sc[j] = n < N ? half_to_float(scales[n]) : 0.0f;
        sc128[j] = -128.0f * sc[j];                      // exact
    }
    f32x16 acc[kIB][2];
#pragma unroll
    for (int i = 0; i < kIB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    // one 32-wide K block of the stage at la / lb: 16 MFMAs per wavefront.  Every fragment is read
    // first and the MFMAs go over all eight accumulators before one is used again (2-3% faster
    // than reading the X fragments block row by block row).
    auto block = [&](const uint8_t* la, const uint8_t* lb, int kb) {
        bf16x8 fa[kIB][2];                               // [i][t]
        bf16x8 fb[2][2];                                 // [j][t]
#pragma unroll
        for (int i = 0; i < kIB; ++i) {
            const int r = wm + 32 * i + r32;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int g = 4 * kb + 2 * h + t;
                fa[i][t] = *reinterpret_cast<const bf16x8*>(la + (r * 8 + (g ^ swz_a(r))) * 16);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = wn + 32 * j + r32;
            const int g = 2 * kb + h;
            const u32x4 q = *reinterpret_cast<const u32x4*>(lb + (r * 4 + (g ^ swz_b(r))) * 16);
            codes_to_bf16(q, sc[j], sc128[j], fb[j][0], fb[j][1]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < kIB; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][t], fb[j][t], acc[i][j], 0, 0, 0);
    };
    // stage st: wait for its loads, then the barrier after which every wave's loads of st are in
    // LDS and every wave is done reading the other buffer, which the next stage's loads then fill
    auto enter = [&](int st) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        if (st + 1 < nst) issue(st + 1);
    };

    if (nst > 0) issue(0);
    const int nfull = (int)(K / kTK);                    // stages with both 32-wide blocks in range
    for (int st = 0; st < nfull; ++st) {
        enter(st);
        const uint8_t* la = lds + (st & 1) * (kAS + kBS);
        block(la, la + kAS, 0);
        block(la, la + kAS, 1);
    }
    const int ktail = (int)(K % kTK);                    // 0, 16, 32 or 48
    if (ktail) {
        enter(nfull);
        const uint8_t* la = lds + (nfull & 1) * (kAS + kBS);
        block(la, la + kAS, 0);
        if (ktail > 32) block(la, la + kAS, 1);
    }

    // Y through an LDS transpose, one 32-row block at a time: 16-byte non-temporal stores of 4
    // consecutive fp32 columns (one wavefront instruction covers 4 rows x 256 bytes), or of 8
    // consecutive bf16 columns (2 rows x 128 bytes), when yvec says that Y rows are 16-byte
    // storable (a 16-byte aligned Y and ldy % 4 == 0 for fp32, ldy % 8 == 0 for bf16); element
    // stores otherwise and at a ragged N edge.  Y is written once and never read here.
    float* tl = reinterpret_cast<float*>(lds) + wave * (32 * 68);   // rows padded to 68 floats
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kIB; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                tl[(8 * (r >> 2) + 4 * h + (r & 3)) * 68 + 32 * j + r32] = acc[i][j][r];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if constexpr (sizeof(YT) == 2) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = lane + 64 * q;
                const int rr = c >> 3, ch = c & 7;
                const f32x4 v0 = *reinterpret_cast<const f32x4*>(tl + rr * 68 + 8 * ch);
                const f32x4 v1 = *reinterpret_cast<const f32x4*>(tl + rr * 68 + 8 * ch + 4);
                const int64_t row = m0 + wm + 32 * i + rr;
                const int64_t col = n0 + wn + 8 * ch;
                if (row < M) {
                    GLB uint16_t* py = (GLB uint16_t*)y + row * ldy + col;
                    if (yvec && col + 8 <= N) {
                        const u32x4 w = {pk_bf16(v0[0], v0[1]), pk_bf16(v0[2], v0[3]), pk_bf16(v1[0], v1[1]),
                                         pk_bf16(v1[2], v1[3])};
                        __builtin_nontemporal_store(w, (GLB u32x4*)py);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (col + e < N) __builtin_nontemporal_store(to_bf16(e < 4 ? v0[e] : v1[e - 4]), py + e);
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            continue;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int c = lane + 64 * q;
            const int rr = c >> 4, ch = c & 15;
            const f32x4 v = *reinterpret_cast<const f32x4*>(tl + rr * 68 + 4 * ch);
            const int64_t row = m0 + wm + 32 * i + rr;
            const int64_t col = n0 + wn + 4 * ch;
            if (row < M) {
                GLB float* py = (GLB float*)y + row * ldy + col;
                if (yvec && col + 4 <= N) {
                    __builtin_nontemporal_store(v, (GLB f32x4*)py);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < N) __builtin_nontemporal_store(v[e], py + e);
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

}  // namespace

int launch_qgemm(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* codes, int64_t ldc,
                 const uint16_t* scales, int64_t N, void* y, int64_t ldy, bool ybf16, uint32_t flags, void* stream)
{
    // the main kernel: 16-byte loadable X and code rows (flags bits 0, 1), K a positive multiple of
    // 16, and a tile's rows of either operand within a 31-bit buffer range.  The choice does not
    // depend on Y, so that both Y types accumulate alike; Y's 16-byte stores follow flags bit 2.
    const bool main = (flags & 3u) == 3u && K > 0 && K % 16 == 0 && ldx < ((int64_t)1 << 21) &&
                      ldc < ((int64_t)1 << 23);
    if (main) {
        const uint64_t tiles = (uint64_t)((N + kTN - 1) / kTN) * (uint64_t)((M + kTM - 1) / kTM);
        if (tiles > 0xFFFFFFFFull) return (int)hipErrorInvalidValue;
        int32_t yvec = (flags & 4u) ? 1 : 0;
        void* args[] = {&x, &M, &K, &ldx, &codes, &ldc, &scales, &N, &y, &ldy, &yvec};
        const void* k = ybf16 ? reinterpret_cast<const void*>(&pgq_qgemm_kernel<uint16_t>)
                              : reinterpret_cast<const void*>(&pgq_qgemm_kernel<float>);
        return (int)launch_plain(k, dim3((unsigned)tiles), dim3(256), args, stream);
    }
    const uint64_t tiles = (uint64_t)((N + kBN - 1) / kBN) * (uint64_t)((M + kBM - 1) / kBM);
    if (tiles > 0xFFFFFFFFull) return (int)hipErrorInvalidValue;
    void* args[] = {&x, &M, &K, &ldx, &codes, &ldc, &scales, &N, &y, &ldy, &flags};
    const void* k = ybf16 ? reinterpret_cast<const void*>(&pgq_qgemm_generic_kernel<uint16_t>)
                          : reinterpret_cast<const void*>(&pgq_qgemm_generic_kernel<float>);
    return (int)launch_plain(k, dim3((unsigned)tiles), dim3(256), args, stream);
}

}  // namespace pgq
